// abi.cpp -- the C ABI: argument checks, workspace layout, launch order.
//
// Nothing here allocates, frees or synchronises; all work goes on the
// caller's stream.  See include/dsa_indexer.h for the contract.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/dsa_indexer.h"
#include "../../include/dsa_indexer_profile.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(int dtype) { return dtype == DSA_BF16 ? 2 : 1; }

struct Range {
  uintptr_t lo, hi;
};
Range span(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + bytes};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_inputs(const dsa_indexer_inputs* in) {
  if (!in) return fail(DSA_ERR_INVALID_ARG, "inputs struct is NULL");
  if (in->batch < 1 || in->num_q < 1 || in->num_k < 1)
    return fail(DSA_ERR_INVALID_ARG, "batch, num_q and num_k must be >= 1");
  if (in->heads != 64) return fail(DSA_ERR_UNSUPPORTED, "heads must be 64");
  if (in->head_dim != 128) return fail(DSA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (in->dtype != DSA_BF16 && in->dtype != DSA_FP8_E4M3) return fail(DSA_ERR_UNSUPPORTED, "unknown dtype");
  if (!in->q || !in->k || !in->w || !in->positions) return fail(DSA_ERR_INVALID_ARG, "q, k, w, positions required");
  if (in->dtype == DSA_FP8_E4M3) {
    if (!in->q_scale || !in->k_scale) return fail(DSA_ERR_INVALID_ARG, "fp8 inputs need q_scale and k_scale");
  } else if (in->q_scale || in->k_scale) {
    return fail(DSA_ERR_INVALID_ARG, "bf16 inputs take no scales");
  }
  const void* ptrs[] = {in->q, in->k, in->w, in->positions, in->q_scale, in->k_scale};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "input pointers must be 16-byte aligned");
  const uint64_t rows = (uint64_t)in->batch * in->num_q;
  if (rows > (1ull << 31) || (uint64_t)in->batch * in->num_k > (1ull << 40))
    return fail(DSA_ERR_INVALID_ARG, "problem too large");
  if (in->flags & ~(uint32_t)(DSA_FLAG_ROUTE_STREAM | DSA_FLAG_ROUTE_SPLIT))
    return fail(DSA_ERR_INVALID_ARG, "unknown flag bits");
  if ((in->flags & DSA_FLAG_ROUTE_STREAM) && (in->flags & DSA_FLAG_ROUTE_SPLIT))
    return fail(DSA_ERR_INVALID_ARG, "DSA_FLAG_ROUTE_STREAM and DSA_FLAG_ROUTE_SPLIT are exclusive");
  return DSA_OK;
}

dsa::Problem problem_of(const dsa_indexer_inputs* in) {
  return dsa::Problem{in->batch,
                      in->num_q,
                      in->num_k,
                      in->dtype,
                      static_cast<const uint8_t*>(in->q),
                      static_cast<const uint8_t*>(in->k),
                      in->w,
                      in->q_scale,
                      in->k_scale,
                      in->positions};
}

// Input byte ranges, for output-aliasing checks.
int check_no_alias(const dsa_indexer_inputs* in, Range out) {
  const size_t eb = elem_bytes(in->dtype);
  const uint64_t B = in->batch, Q = in->num_q, N = in->num_k;
  Range r[] = {span(in->q, B * Q * 64 * 128 * eb), span(in->k, B * N * 128 * eb), span(in->w, B * Q * 64 * 4),
               span(in->positions, B * Q * 4)};
  for (const Range& x : r)
    if (overlaps(x, out)) return fail(DSA_ERR_INVALID_ARG, "an output aliases an input");
  if (in->q_scale && overlaps(span(in->q_scale, B * Q * 4), out))
    return fail(DSA_ERR_INVALID_ARG, "an output aliases an input");
  if (in->k_scale && overlaps(span(in->k_scale, B * N * 4), out))
    return fail(DSA_ERR_INVALID_ARG, "an output aliases an input");
  return DSA_OK;
}

int check_topk(int32_t topk) {
  if (topk < 1) return fail(DSA_ERR_INVALID_ARG, "topk must be >= 1");
  if (topk > 4096) return fail(DSA_ERR_UNSUPPORTED, "topk must be <= 4096");
  return DSA_OK;
}

// Few query-row groups cannot fill the GPU with one workgroup per 8 rows:
// such calls (decode) score rows split across the key axis into a stored
// [B*Q, N] row block and select from it.  The caller's flags can pin either
// route.
bool use_split_rows(const dsa_indexer_inputs* in) {
  if (in->flags & DSA_FLAG_ROUTE_SPLIT) return true;
  if (in->flags & DSA_FLAG_ROUTE_STREAM) return false;
  const uint64_t groups = (uint64_t)in->batch * ((in->num_q + 7) / 8);
  const uint64_t row_bytes = (uint64_t)in->batch * in->num_q * in->num_k * 4;
  return groups < 256 && row_bytes <= (8ull << 30);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t topk_workspace(const dsa_indexer_inputs* in, int32_t topk) {
  const uint64_t rows = (uint64_t)in->batch * in->num_q;
  if (use_split_rows(in)) return round_up(rows * in->num_k * 4, 256) + rows * dsa::kRowHistBins * 4;
  return round_up(rows * (uint64_t)dsa::stream_capacity(topk) * 8, 256);
}

int hip_status(hipError_t e) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, std::string("HIP launch failed: ") + hipGetErrorString(e));
  return DSA_OK;
}

int run_topk(const dsa_indexer_inputs* in, int32_t topk, int32_t* out_idx, float* out_score, void* workspace,
             hipStream_t st) {
  const dsa::Problem p = problem_of(in);
  if (use_split_rows(in)) {
    float* rows = static_cast<float*>(workspace);
    const uint64_t nrows = (uint64_t)in->batch * in->num_q;
    uint32_t* hist = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) +
                                                 round_up(nrows * in->num_k * 4, 256));
    int rc = hip_status(dsa::launch_scores(p, rows, hist, st));
    if (rc) return rc;
    return hip_status(dsa::launch_select_rows(p, rows, hist, topk, out_idx, out_score, st));
  }
  return hip_status(dsa::launch_topk_stream(p, topk, dsa::stream_capacity(topk), static_cast<uint64_t*>(workspace),
                                            out_idx, out_score, st));
}

int check_topk_outputs(const dsa_indexer_inputs* in, int32_t topk, int32_t* out_idx, float* out_score,
                       void* workspace, size_t workspace_bytes, size_t need) {
  if (!out_idx) return fail(DSA_ERR_INVALID_ARG, "out_idx is required");
  if (!aligned16(out_idx) || (out_score && !aligned16(out_score)))
    return fail(DSA_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  const uint64_t n = (uint64_t)in->batch * in->num_q * topk;
  int rc = check_no_alias(in, span(out_idx, n * 4));
  if (rc) return rc;
  if (out_score) {
    if ((rc = check_no_alias(in, span(out_score, n * 4)))) return rc;
    if (overlaps(span(out_idx, n * 4), span(out_score, n * 4)))
      return fail(DSA_ERR_INVALID_ARG, "out_idx and out_score overlap");
  }
  if (workspace_bytes < need || (need && !workspace))
    return fail(DSA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  if (need && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (need) {
    Range ws = span(workspace, need);
    if ((rc = check_no_alias(in, ws))) return rc;
    if (overlaps(ws, span(out_idx, n * 4)) || (out_score && overlaps(ws, span(out_score, n * 4))))
      return fail(DSA_ERR_INVALID_ARG, "workspace overlaps an output");
  }
  return DSA_OK;
}


// ---------------------------------------------------------------- pruned path

struct PruneConfig {
  int num_seeds;
  int num_retained;
  const int32_t* seed_idx;
  const uint8_t* force_recover;
  bool raised_start;
  bool compact;
  bool anchor;
};

int prune_config(const dsa_prune_opts* o, PruneConfig* pc) {
  const uint32_t flags = o ? o->flags : 0u;
  if (flags & ~(uint32_t)(DSA_PRUNE_START_AT_TAU | DSA_PRUNE_COMPACT_RECORDS | DSA_PRUNE_ANCHOR_SEEDS))
    return fail(DSA_ERR_INVALID_ARG, "unknown pruning flags");
  pc->anchor = (flags & DSA_PRUNE_ANCHOR_SEEDS) != 0;
  // anchor seeds are no even sample of the keys: every row starts at tau
  pc->raised_start = !(flags & DSA_PRUNE_START_AT_TAU) && !pc->anchor;
  pc->compact = (flags & DSA_PRUNE_COMPACT_RECORDS) != 0;
  pc->num_seeds = (o && o->num_seeds) ? o->num_seeds : 12288;
  pc->num_retained = (o && o->num_retained) ? o->num_retained : 30;
  pc->seed_idx = o ? o->seed_idx : nullptr;
  pc->force_recover = o ? o->force_recover : nullptr;
  if (pc->num_seeds < 1 || pc->num_seeds > (1 << 26)) return fail(DSA_ERR_INVALID_ARG, "num_seeds out of range");
  if (o && o->seed_idx && o->num_seeds < 1) return fail(DSA_ERR_INVALID_ARG, "seed_idx needs num_seeds > 0");
  if (pc->num_retained < 1 || pc->num_retained > 30)
    return fail(DSA_ERR_UNSUPPORTED, "num_retained must be in 1..30");
  if (pc->seed_idx && !aligned16(pc->seed_idx)) return fail(DSA_ERR_INVALID_ARG, "seed_idx must be 16-byte aligned");
  if (pc->anchor && pc->seed_idx) return fail(DSA_ERR_INVALID_ARG, "anchor seeds and seed_idx exclude each other");
  return DSA_OK;
}

// Compact records keep the key index in the low bits of 32: at most 24 of
// them, so that the score code keeps at least 8.
int check_prune_fit(const dsa_indexer_inputs* in, const PruneConfig& pc, int32_t topk) {
  if (pc.compact && in->num_k > (1 << 24))
    return fail(DSA_ERR_UNSUPPORTED, "compact records need num_k <= 2^24");
  if (pc.anchor && pc.num_seeds < topk) return fail(DSA_ERR_INVALID_ARG, "anchor seeds need num_seeds >= topk");
  return DSA_OK;
}

// Anchor rows per sequence: num_seeds / topk, at least 1, at most Q.
int anchor_count(const dsa_indexer_inputs* in, const PruneConfig& pc, int32_t topk) {
  return std::min(in->num_q, std::max(1, pc.num_seeds / topk));
}

// Workspace carve-up of the pruned path; returns the total bytes.  With a
// base pointer it also fills the buffer pointers.
size_t pruned_layout(const dsa_indexer_inputs* in, int32_t topk, const PruneConfig& pc, uint8_t* base,
                     dsa::PrunedBuffers* pb, uint64_t** cand = nullptr) {
  const uint64_t R = (uint64_t)in->batch * in->num_q, B = in->batch, N = in->num_k;
  const uint64_t words = (N + 31) / 32;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return base ? base + o : nullptr;
  };
  uint8_t* c = take(R * (uint64_t)dsa::stream_capacity(topk) * 8);
  uint8_t* rows = take(R * 32 * 128 * elem_bytes(in->dtype));
  uint8_t* coef = take(R * 32 * 4);
  uint8_t* misc = take(R * 4 * 4);
  uint8_t* flag = take(R * 4);
  uint8_t* kn = take(B * N * 4);
  uint8_t* seeds = take(B * (uint64_t)pc.num_seeds * 4);
  uint8_t* scount = take(B * 4);
  uint8_t* bits = take(B * words * 4);
  uint8_t* bflag = take(B * 4);
  uint8_t* skeys = take(B * (uint64_t)pc.num_seeds * 128 * elem_bytes(in->dtype));
  uint8_t* sksc = take(B * (uint64_t)pc.num_seeds * 4);
  uint8_t* spos = take(R * 4);
  uint8_t* stidx = take(R * (uint64_t)topk * 4);
  uint8_t* stsc = take(R * (uint64_t)topk * 4);
  const uint64_t mwords = (uint64_t)dsa::prune_mask_words(in->num_k, 128 * (int)elem_bytes(in->dtype));
  uint8_t* ctl = take(R * sizeof(dsa::PruneRowCtl));
  uint8_t* hist = take(R * 256 * 4);
  uint8_t* mask = take(R * mwords * 8);
  if (base && pb) {
    if (cand) *cand = reinterpret_cast<uint64_t*>(c);
    pb->plan_rows = rows;
    pb->plan_coef = reinterpret_cast<float*>(coef);
    pb->plan_misc = reinterpret_cast<float*>(misc);
    pb->plan_flag = reinterpret_cast<int32_t*>(flag);
    pb->knorm = reinterpret_cast<float*>(kn);
    pb->seeds = reinterpret_cast<int32_t*>(seeds);
    pb->seed_count = reinterpret_cast<int32_t*>(scount);
    pb->seed_stride = pc.num_seeds;
    pb->seed_bits = reinterpret_cast<uint32_t*>(bits);
    pb->bits_stride = (int)words;
    pb->batch_flag = reinterpret_cast<int32_t*>(bflag);
    pb->seed_keys = skeys;
    pb->seed_kscale = reinterpret_cast<float*>(sksc);
    pb->seed_pos = reinterpret_cast<int32_t*>(spos);
    pb->seed_top_idx = reinterpret_cast<int32_t*>(stidx);
    pb->seed_top_score = reinterpret_cast<float*>(stsc);
    pb->ctl = reinterpret_cast<dsa::PruneRowCtl*>(ctl);
    pb->hist = reinterpret_cast<uint32_t*>(hist);
    pb->mask = reinterpret_cast<uint64_t*>(mask);
    pb->mask_stride = (int)mwords;
  }
  return off;
}


// ---------------------------------------------------------------- projections

int check_proj_inputs(const dsa_proj_inputs* in) {
  if (!in) return fail(DSA_ERR_INVALID_ARG, "projection inputs struct is NULL");
  if (in->num_tokens < 1 || in->num_tokens > (1 << 22))
    return fail(DSA_ERR_INVALID_ARG, "num_tokens must be in 1..4194304");
  if (in->heads != 64) return fail(DSA_ERR_UNSUPPORTED, "heads must be 64");
  if (in->head_dim != 128) return fail(DSA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (in->hidden < 8 || in->hidden > 65536 || in->hidden % 8 || in->q_latent < 8 || in->q_latent > 65536 ||
      in->q_latent % 8)
    return fail(DSA_ERR_INVALID_ARG, "hidden and q_latent must be multiples of 8 in 8..65536");
  if (in->block_tokens != 0 && (in->block_tokens < 64 || in->block_tokens > (1 << 18)))
    return fail(DSA_ERR_INVALID_ARG, "block_tokens must be 0 or in 64..262144");
  const void* ptrs[] = {in->c_q, in->x, in->w_iq, in->w_ik, in->w_iw};
  for (const void* p : ptrs) {
    if (!p) return fail(DSA_ERR_INVALID_ARG, "c_q, x, w_iq, w_ik, w_iw are required");
    if (!aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "input pointers must be 16-byte aligned");
  }
  return DSA_OK;
}

int check_proj_no_alias(const dsa_proj_inputs* in, Range out) {
  const uint64_t T = in->num_tokens, D = in->hidden, L = in->q_latent;
  const Range r[] = {span(in->c_q, T * L * 2), span(in->x, T * D * 2), span(in->w_iq, 8192 * L * 2),
                     span(in->w_ik, 128 * D * 2), span(in->w_iw, 64 * D * 2)};
  for (const Range& x : r)
    if (overlaps(x, out)) return fail(DSA_ERR_INVALID_ARG, "an output aliases an input");
  return DSA_OK;
}

// ---------------------------------------------------------------- sparse MLA

int check_mla_inputs(const dsa_mla_inputs* in) {
  if (!in) return fail(DSA_ERR_INVALID_ARG, "attention inputs struct is NULL");
  if (in->batch < 1 || in->num_q < 1 || in->num_k < 1)
    return fail(DSA_ERR_INVALID_ARG, "batch, num_q and num_k must be >= 1");
  if (in->heads != 128) return fail(DSA_ERR_UNSUPPORTED, "heads must be 128");
  if (in->latent_dim != 512 || in->rope_dim != 64)
    return fail(DSA_ERR_UNSUPPORTED, "latent_dim must be 512 and rope_dim 64");
  if (in->topk < 1) return fail(DSA_ERR_INVALID_ARG, "topk must be >= 1");
  if (in->topk > 2048) return fail(DSA_ERR_UNSUPPORTED, "topk must be <= 2048");
  if (in->num_splits < 0 || in->num_splits > 8) return fail(DSA_ERR_INVALID_ARG, "num_splits must be in 0..8");
  const void* ptrs[] = {in->q, in->kv, in->indices};
  for (const void* p : ptrs) {
    if (!p) return fail(DSA_ERR_INVALID_ARG, "q, kv and indices are required");
    if (!aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "input pointers must be 16-byte aligned");
  }
  if (in->page_table) {
    if (!aligned16(in->page_table)) return fail(DSA_ERR_INVALID_ARG, "page_table must be 16-byte aligned");
    if (in->page_size < 1 || in->num_pages < 1 || in->pages_per_seq < 1)
      return fail(DSA_ERR_INVALID_ARG, "page_size, pages_per_seq and num_pages must be >= 1");
    if ((uint64_t)in->pages_per_seq * in->page_size < (uint64_t)in->num_k)
      return fail(DSA_ERR_INVALID_ARG, "pages_per_seq * page_size must cover num_k");
    if ((uint64_t)in->num_pages * in->page_size > (1ull << 31))
      return fail(DSA_ERR_INVALID_ARG, "num_pages * page_size must be <= 2^31");
  }
  const uint64_t rows = (uint64_t)in->batch * in->num_q;
  if (rows > (1ull << 31) || (uint64_t)in->batch * in->num_k > (1ull << 40))
    return fail(DSA_ERR_INVALID_ARG, "problem too large");
  return DSA_OK;
}

// Workspace of the sparse MLA call: per work unit (a row, or a row's tile
// range when rows are few) the head maxima and a retry flag, and for split
// rows the partial outputs and (reference, weight sum) pairs.
struct MlaLayout {
  int nsplit;
  size_t row_max, retry, part_o, part_ml, total;
};
MlaLayout mla_layout(const dsa_mla_inputs* in) {
  const uint64_t rows = (uint64_t)in->batch * in->num_q;
  MlaLayout L{};
  L.nsplit = dsa::mla_splits((int)rows, in->num_splits);
  const uint64_t units = rows * L.nsplit;
  size_t off = 0;
  L.row_max = off;
  off += round_up(units * 128 * 4, 256);
  L.retry = off;
  off += round_up(units * 4, 256);
  L.part_o = off;
  if (L.nsplit > 1) off += round_up(units * 128 * 512 * 4, 256);
  L.part_ml = off;
  if (L.nsplit > 1) off += round_up(units * 128 * 2 * 4, 256);
  L.total = off;
  return L;
}
size_t mla_workspace(const dsa_mla_inputs* in) { return mla_layout(in).total; }
}  // namespace

extern "C" {

int dsa_indexer_scores(const dsa_indexer_inputs* in, float* scores, void* stream) {
  int rc = check_inputs(in);
  if (rc) return rc;
  if (!scores) return fail(DSA_ERR_INVALID_ARG, "scores output is required");
  if (!aligned16(scores)) return fail(DSA_ERR_INVALID_ARG, "scores must be 16-byte aligned");
  if ((rc = check_no_alias(in, span(scores, (uint64_t)in->batch * in->num_q * in->num_k * 4)))) return rc;
  return hip_status(dsa::launch_scores(problem_of(in), scores, nullptr, static_cast<hipStream_t>(stream)));
}

int dsa_indexer_topk(const dsa_indexer_inputs* in, int32_t topk, int32_t* out_idx, float* out_score,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_inputs(in);
  if (rc) return rc;
  if ((rc = check_topk(topk))) return rc;
  const size_t need = topk_workspace(in, topk);
  if ((rc = check_topk_outputs(in, topk, out_idx, out_score, workspace, workspace_bytes, need))) return rc;
  return run_topk(in, topk, out_idx, out_score, workspace, static_cast<hipStream_t>(stream));
}

int dsa_indexer_topk_noalloc(const dsa_indexer_inputs* in, int32_t topk, int32_t* out_idx, float* out_score,
                             void* stream) {
  int rc = check_inputs(in);
  if (rc) return rc;
  if ((rc = check_topk(topk))) return rc;
  const size_t need = topk_workspace(in, topk);
  if (need > dsa::kNoAllocScratchBytes)
    return fail(DSA_ERR_WORKSPACE, "call needs " + std::to_string(need) + " bytes of scratch; the fixed scratch holds " +
                                       std::to_string(dsa::kNoAllocScratchBytes));
  void* ws = nullptr;
  std::string err;
  if (dsa::noalloc_scratch(&ws, &err)) return fail(DSA_ERR_HIP, err);
  if ((rc = check_topk_outputs(in, topk, out_idx, out_score, ws, dsa::kNoAllocScratchBytes, need))) return rc;
  return run_topk(in, topk, out_idx, out_score, ws, static_cast<hipStream_t>(stream));
}

size_t dsa_indexer_workspace_bytes(int op, const dsa_indexer_inputs* in, int32_t topk, const dsa_prune_opts* opts) {
  g_last_error.clear();
  if (check_inputs(in)) return 0;
  if (op == DSA_OP_SCORES) return 0;
  if (check_topk(topk)) return 0;
  if (op == DSA_OP_TOPK) return topk_workspace(in, topk);
  if (op == DSA_OP_TOPK_PRUNED) {
    PruneConfig pc;
    if (prune_config(opts, &pc) || check_prune_fit(in, pc, topk)) return 0;
    return pruned_layout(in, topk, pc, nullptr, nullptr);
  }
  fail(DSA_ERR_INVALID_ARG, "unknown op");
  return 0;
}

int dsa_indexer_topk_pruned(const dsa_indexer_inputs* in, int32_t topk, const dsa_prune_opts* opts,
                            int32_t* out_idx, float* out_score, const dsa_prune_stats* stats, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int rc = check_inputs(in);
  if (rc) return rc;
  if ((rc = check_topk(topk))) return rc;
  PruneConfig pc;
  if ((rc = prune_config(opts, &pc))) return rc;
  if ((rc = check_prune_fit(in, pc, topk))) return rc;
  const size_t need = pruned_layout(in, topk, pc, nullptr, nullptr);
  if ((rc = check_topk_outputs(in, topk, out_idx, out_score, workspace, workspace_bytes, need))) return rc;
  if (stats) {
    const uint64_t rows = (uint64_t)in->batch * in->num_q;
    const Range outs[] = {span(stats->tau, rows * 4),
                          span(stats->screened, rows * 4),
                          span(stats->survivors, rows * 4),
                          span(stats->recovered, rows),
                          span(stats->upper_bound, rows * in->num_k * 4),
                          span(stats->plan_rows, rows * 32 * 128 * elem_bytes(in->dtype)),
                          span(stats->plan_coef, rows * 32 * 4),
                          span(stats->plan_misc, rows * 2 * 4)};
    const void* ptrs[] = {stats->tau,         stats->screened,  stats->survivors, stats->recovered,
                          stats->upper_bound, stats->plan_rows, stats->plan_coef, stats->plan_misc};
    for (int i = 0; i < 8; ++i) {
      if (!ptrs[i]) continue;
      if ((rc = check_no_alias(in, outs[i]))) return rc;
      if (overlaps(outs[i], span(workspace, need))) return fail(DSA_ERR_INVALID_ARG, "stats overlap the workspace");
    }
  }
  dsa::PrunedBuffers pb{};
  uint64_t* cand = nullptr;
  pruned_layout(in, topk, pc, static_cast<uint8_t*>(workspace), &pb, &cand);
  pb.raised_start = pc.raised_start ? 1 : 0;
  pb.compact = pc.compact ? 1 : 0;
  if (stats) {
    pb.st_tau = stats->tau;
    pb.st_screened = stats->screened;
    pb.st_surv = stats->survivors;
    pb.st_rec = stats->recovered;
    pb.st_ub = stats->upper_bound;
  }
  const dsa::Problem p = problem_of(in);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pc.anchor) {
    // seeds from anchor queries: the anchor rows' exact Top-K by the
    // unpruned streaming path (into their rows of the seed Top-K buffer; the
    // planner's row flags serve as the row mask until the planner writes
    // them), then the distinct keys of those sets
    const int A = anchor_count(in, pc, topk);
    if ((rc = hip_status(dsa::launch_anchor_rows(p, A, pb.plan_flag, st)))) return rc;
    if ((rc = hip_status(dsa::launch_topk_stream_rows(p, topk, dsa::stream_capacity(topk), cand, pb.seed_top_idx,
                                                      pb.seed_top_score, pb.plan_flag, "k_topk_stream_anchors", st))))
      return rc;
    if ((rc = hip_status(dsa::launch_anchor_seeds(p, A, topk, pb.seed_top_idx, pb.seed_stride, pb.seeds,
                                                  pb.seed_count, pb.seed_bits, pb.batch_flag, st))))
      return rc;
  } else if ((rc = hip_status(dsa::launch_seed_prep(p, pc.num_seeds, pc.seed_idx, pb.seeds, pb.seed_count,
                                                    pb.seed_bits, pb.batch_flag, st)))) {
    return rc;
  }
  if ((rc = hip_status(dsa::launch_key_norms(p, pb.knorm, st)))) return rc;
  // the seeds' exact Top-K per row: the streaming Top-K over the packed seed
  // keys (the same score routine, so the same scores)
  if ((rc = hip_status(dsa::launch_seed_pack(p, pb.seeds, pb.seed_count, pb.seed_stride, pb.seed_keys,
                                             pb.seed_kscale, pb.seed_pos, st))))
    return rc;
  {
    dsa::Problem sp = p;
    sp.N = pb.seed_stride;
    sp.k = pb.seed_keys;
    sp.k_scale = in->dtype == DSA_BF16 ? nullptr : pb.seed_kscale;
    sp.pos = pb.seed_pos;
    if ((rc = hip_status(dsa::launch_topk_stream(sp, topk, dsa::stream_capacity(topk), cand, pb.seed_top_idx,
                                                 pb.seed_top_score, st))))
      return rc;
  }
  if ((rc = hip_status(dsa::launch_plan(p, pc.num_retained, pb.seeds, pb.seed_count, pb.seed_stride, pb.batch_flag,
                                        pc.force_recover, pb.plan_rows, pb.plan_coef, pb.plan_misc, pb.plan_flag,
                                        st))))
    return rc;
  if (stats && (stats->plan_rows || stats->plan_coef || stats->plan_misc)) {  // debug export of the plans
    const uint64_t rows = (uint64_t)in->batch * in->num_q;
    if (stats->plan_rows &&
        (rc = hip_status(hipMemcpyAsync(stats->plan_rows, pb.plan_rows, rows * 32 * 128 * elem_bytes(in->dtype),
                                        hipMemcpyDeviceToDevice, st))))
      return rc;
    if (stats->plan_coef &&
        (rc = hip_status(hipMemcpyAsync(stats->plan_coef, pb.plan_coef, rows * 32 * 4, hipMemcpyDeviceToDevice, st))))
      return rc;
    if (stats->plan_misc &&
        (rc = hip_status(hipMemcpy2DAsync(stats->plan_misc, 2 * 4, pb.plan_misc, 4 * 4, 2 * 4, rows,
                                          hipMemcpyDeviceToDevice, st))))
      return rc;
  }
  return hip_status(
      dsa::launch_topk_pruned(p, topk, dsa::stream_capacity(topk), cand, out_idx, out_score, pb, st));
}

size_t dsa_indexer_project_workspace_bytes(const dsa_proj_inputs* in) {
  g_last_error.clear();
  if (check_proj_inputs(in)) return 0;
  return dsa::proj_workspace_bytes(in->num_tokens, in->hidden, in->block_tokens);
}

int dsa_indexer_project(const dsa_proj_inputs* in, int32_t out_dtype, void* q_out, float* q_scale, void* k_out,
                        float* k_scale, float* w_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_proj_inputs(in);
  if (rc) return rc;
  int mode;
  if (out_dtype == DSA_FP8_E4M3)
    mode = 0;
  else if (out_dtype == DSA_BF16)
    mode = 1;
  else if (out_dtype == DSA_F32)
    mode = 2;
  else
    return fail(DSA_ERR_UNSUPPORTED, "out_dtype must be DSA_FP8_E4M3, DSA_BF16 or DSA_F32");
  if (!q_out || !k_out || !w_out) return fail(DSA_ERR_INVALID_ARG, "q_out, k_out and w_out are required");
  if (mode == 0 && (!q_scale || !k_scale)) return fail(DSA_ERR_INVALID_ARG, "fp8 outputs need q_scale and k_scale");
  if (mode != 0 && (q_scale || k_scale)) return fail(DSA_ERR_INVALID_ARG, "only fp8 outputs take scales");
  const void* outs_p[] = {q_out, k_out, w_out, q_scale, k_scale};
  for (const void* p : outs_p)
    if (p && !aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  const uint64_t T = in->num_tokens;
  const uint64_t eb = mode == 0 ? 1 : mode == 1 ? 2 : 4;
  const size_t need = dsa::proj_workspace_bytes(in->num_tokens, in->hidden, in->block_tokens);
  if (workspace_bytes < need || !workspace)
    return fail(DSA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const Range outs[] = {span(q_out, T * 8192 * eb), span(k_out, T * 128 * eb), span(w_out, T * 64 * 4),
                        span(q_scale, q_scale ? T * 4 : 0), span(k_scale, k_scale ? T * 4 : 0),
                        span(workspace, need)};
  for (int i = 0; i < 6; ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    if ((rc = check_proj_no_alias(in, outs[i]))) return rc;
    for (int j = 0; j < i; ++j)
      if (outs[j].lo != outs[j].hi && overlaps(outs[i], outs[j]))
        return fail(DSA_ERR_INVALID_ARG, "outputs and workspace must not overlap");
  }
  const dsa::ProjProblem p{in->num_tokens,
                           in->hidden,
                           in->q_latent,
                           in->block_tokens,
                           static_cast<const uint16_t*>(in->c_q),
                           static_cast<const uint16_t*>(in->x),
                           static_cast<const uint16_t*>(in->w_iq),
                           static_cast<const uint16_t*>(in->w_ik),
                           static_cast<const uint16_t*>(in->w_iw)};
  std::string err;
  const int prc = dsa::run_projection(p, mode, static_cast<uint8_t*>(q_out), q_scale, static_cast<uint8_t*>(k_out),
                                      k_scale, w_out, static_cast<uint8_t*>(workspace),
                                      static_cast<hipStream_t>(stream), &err);
  if (prc == 2) return fail(DSA_ERR_UNSUPPORTED, err);
  if (prc) return fail(DSA_ERR_HIP, err);
  return DSA_OK;
}

size_t dsa_sparse_mla_workspace_bytes(const dsa_mla_inputs* in) {
  g_last_error.clear();
  if (check_mla_inputs(in)) return 0;
  return mla_workspace(in);
}

int dsa_sparse_mla(const dsa_mla_inputs* in, float sm_scale, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc = check_mla_inputs(in);
  if (rc) return rc;
  if (!(sm_scale >= 0.0f) || !(sm_scale < INFINITY)) return fail(DSA_ERR_INVALID_ARG, "sm_scale must be finite and >= 0");
  if (!out) return fail(DSA_ERR_INVALID_ARG, "out is required");
  if (!aligned16(out) || (lse && !aligned16(lse))) return fail(DSA_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  const size_t need = mla_workspace(in);
  if (workspace_bytes < need || !workspace)
    return fail(DSA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const uint64_t rows = (uint64_t)in->batch * in->num_q, B = in->batch, N = in->num_k;
  const uint64_t kv_rows = in->page_table ? (uint64_t)in->num_pages * in->page_size : B * N;
  const Range inputs[] = {span(in->q, rows * 128 * 576 * 2), span(in->kv, kv_rows * 576 * 2),
                          span(in->indices, rows * (uint64_t)in->topk * 4),
                          span(in->page_table, in->page_table ? B * (uint64_t)in->pages_per_seq * 4 : 0)};
  const Range outs[] = {span(out, rows * 128 * 512 * 2), span(lse, lse ? rows * 128 * 4 : 0), span(workspace, need)};
  for (int i = 0; i < 3; ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    for (const Range& x : inputs)
      if (overlaps(x, outs[i])) return fail(DSA_ERR_INVALID_ARG, "an output aliases an input");
    for (int j = 0; j < i; ++j)
      if (outs[j].lo != outs[j].hi && overlaps(outs[i], outs[j]))
        return fail(DSA_ERR_INVALID_ARG, "outputs and workspace must not overlap");
  }
  const dsa::MlaProblem p{in->batch,
                          in->num_q,
                          in->num_k,
                          in->topk,
                          static_cast<const uint16_t*>(in->q),
                          static_cast<const uint16_t*>(in->kv),
                          in->indices,
                          in->page_table,
                          in->page_table ? in->page_size : 1,
                          in->page_table ? in->pages_per_seq : 1,
                          in->page_table ? in->num_pages : 1};
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const MlaLayout L = mla_layout(in);
  return hip_status(dsa::launch_sparse_mla(
      p, sm_scale, static_cast<uint16_t*>(out), lse, reinterpret_cast<float*>(ws + L.row_max),
      reinterpret_cast<int32_t*>(ws + L.retry), L.nsplit, L.nsplit > 1 ? reinterpret_cast<float*>(ws + L.part_o) : nullptr,
      L.nsplit > 1 ? reinterpret_cast<float*>(ws + L.part_ml) : nullptr, static_cast<hipStream_t>(stream)));
}

const char* dsa_indexer_error_string(int code) {
  switch (code) {
    case DSA_OK:
      return "ok";
    case DSA_ERR_INVALID_ARG:
      return "invalid argument";
    case DSA_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case DSA_ERR_WORKSPACE:
      return "workspace too small";
    case DSA_ERR_HIP:
      return "HIP error";
    default:
      return "unknown error";
  }
}

const char* dsa_indexer_last_error(void) { return g_last_error.c_str(); }

int dsa_indexer_mfma_ceiling(int32_t dtype, int32_t mode, int32_t iters, float* out, size_t out_len, void* stream,
                             int32_t* workgroups) {
  if (!workgroups) return fail(DSA_ERR_INVALID_ARG, "workgroups must not be NULL");
  if (dtype != DSA_BF16 && dtype != DSA_FP8_E4M3) return fail(DSA_ERR_INVALID_ARG, "unknown dtype");
  if (mode < 0 || mode > 2) return fail(DSA_ERR_INVALID_ARG, "mode must be 0, 1 or 2");
  if (mode == 2 && dtype != DSA_BF16) return fail(DSA_ERR_INVALID_ARG, "mode 2 is bf16 only");
  if (iters < 2 || (iters & 1)) return fail(DSA_ERR_INVALID_ARG, "iters must be even and >= 2");
  const int wg = dsa::mfma_ceiling_workgroups();
  if (wg < 1) return fail(DSA_ERR_HIP, "device query failed");
  *workgroups = wg;
  if (!out) return DSA_OK;
  if (out_len < (size_t)wg * 256) return fail(DSA_ERR_INVALID_ARG, "out holds fewer than workgroups * 256 floats");
  return hip_status(dsa::launch_mfma_ceiling(dtype, mode, iters, wg, out,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
