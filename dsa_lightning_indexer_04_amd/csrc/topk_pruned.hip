// topk_pruned.hip -- exact Top-K with certified (DoSA) pruning, fused.
//
// Flow per query row (DoSA reading notes, annotation LBKERZAW, steps 1-3;
// 机器之心 DoSA article, sections 03-04, Fig. 2-3):
//   1. seeds: the seed keys are scored with all heads by the same routine as
//      every other path and go into the row's candidate buffer; the K-th best
//      seed record is the threshold tau (K distinct visible keys reach it, so
//      it cannot exceed the true K-th score);
//   2. screen: every other visible key gets the certified upper bound U from
//      16 plan rows (14 retained heads, the folded negative-head row, the
//      linear row; see prune_prep.hip) -- one 16x16 MFMA block per 16 keys --
//      and survives iff its record (U, key) is not below the row's running
//      threshold; a 64-lane ballot packs the survivors into a bitmask;
//   3. compact + refine: survivors are queued per row and rescored with all
//      heads in batches of 32 (keys gathered by index, same score routine),
//      and only records not below the threshold are written as candidates;
//   4. select: the row's candidates (seed Top-K and refined survivors) are cut
//      to the exact Top-K by score, then key index.
// The running threshold starts at tau and only rises when the candidate
// buffer is cut (the K-th best exact score found so far), which is valid for
// the same reason as tau.  The bounds never rank: only exact scores do.
// Recovery: a row flagged by the planner (non-finite plan, forced, invalid
// seeds) lets every key survive, i.e. runs the unpruned computation.
#include <math.h>

#include "kernels.h"
#include "stream_common.h"

namespace dsa {

constexpr int kPlanRowsK = 32;
constexpr int kLinRowK = 31;
constexpr int kAuxRowK = 30;
constexpr int kRetainedK = 30;
constexpr int kCutSlack = 1024;  // records kept beyond topk before the threshold is raised
constexpr int kRing = 6;         // LDS key tiles: the screen's, the next one, and four awaiting refinement
constexpr int kRefineEvery = 4;  // tiles between refine rounds

struct PrunePlan {
  const uint8_t* rows;       // [R][32][128] dtype: bound rows
  const float* coef;         // [R][32]: c_0..c_29, aux multiplier, linear multiplier
  const float* misc;         // [R][4]: kappa, e_neg
  const int32_t* flag;       // [R]: 1 = recover (no pruning)
  const float* knorm;        // [B][N]: |k|, rounded up
  const int32_t* seeds;      // [B][seed_stride] ascending
  const int32_t* seed_count; // [B]
  int seed_stride;
  const uint32_t* seed_bits; // [B][bits_stride]
  int bits_stride;
  float* st_tau;
  int32_t* st_screened;
  int32_t* st_surv;
  uint8_t* st_rec;
  float* st_ub;              // [R][N] debug bounds or null
};

// Append state of one row (all wave-uniform except `rec`/`live`).
struct RowState {
  uint64_t* buf;
  int cnt, nst;
  uint64_t thr;
};

__device__ __forceinline__ void append_rec(RowState& rs, uint64_t rec, bool live, uint64_t* stage, uint32_t* hist,
                                           int topk, int cap, int lane) {
  uint64_t bal = __ballot(live && rec >= rs.thr);
  if (bal) {
    if (rs.cnt + rs.nst + __popcll(bal) > cap) {
      const Cut c = cut_candidates_d8(rs.buf, rs.cnt, stage, rs.nst, hist, topk, topk, lane);
      rs.cnt = c.cnt;
      rs.thr = c.thr;
      rs.nst = 0;
      bal = __ballot(live && rec >= rs.thr);
    }
    if (live && rec >= rs.thr)
      stage[rs.nst + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] =
          rec;
    rs.nst += __popcll(bal);
  }
}

template <int DT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_topk_pruned(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ qsc, const float* __restrict__ ksc, const int32_t* __restrict__ pos, int Q, int N,
    int topk, int cap, uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_score,
    PrunePlan pp) {
  constexpr int RB = Frag<DT>::kRowBytes;
  constexpr int KT = kTileBytes / RB;
  constexpr int NSB = KT / 32;
  __shared__ u32x4 ktile[kRing][kTileChunks];
  __shared__ float kscale_tile[kRing][KT];
  __shared__ uint32_t hist[kWaves][256];  // radix-select bins (8-bit digits)
  __shared__ uint64_t stage[kWaves][KT + 32];
  __shared__ int32_t squeue[kWaves][kRefineEvery * KT];  // survivor list (see below)
  __shared__ float knorm_tile[kRing][KT];
  __shared__ uint32_t sbits_tile[kRing][KT / 32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = gridDim.x - 1 - blockIdx.x;
  const int b = blockIdx.y;
  const int t = group * kWaves + wave;
  const bool valid = t < Q;
  const size_t row = (size_t)b * Q + min(t, Q - 1);
  const int vis = valid ? min(max(pos[row] + 1, 0), N) : 0;
  int wg_vis = 0;
  for (int j = 0; j < kWaves; ++j) {
    const int tj = group * kWaves + j;
    if (tj < Q) wg_vis = max(wg_vis, min(max(pos[(size_t)b * Q + tj] + 1, 0), N));
  }

  // query rows in registers; head weights in LDS (read at each full epilogue)
  __shared__ __align__(16) float wrow[kWaves][kHeads];
  Frag<DT> qa[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) load_frag<DT>(qa[blk], q + (row * kHeads + 32 * blk + (lane & 31)) * RB, lane);
  wrow[wave][lane] = w[row * kHeads + lane];
  const float* my_w = wrow[wave];
  const float qscale = (DT == kFP8) ? qsc[row] : 1.0f;

  // screen side: the 32 plan rows as one 32x32 MFMA A operand; lane l holds
  // rows 8*(v/4) + 4*(l/32) + v%4 of the result (v = 0..15), with their
  // coefficients in cl[v].  Rows 30 (aux) and 31 (linear) land in lanes
  // 32..63 at v = 14, 15; the other lanes get zero multipliers for them.
  Frag<DT> sa;
  load_frag<DT>(sa, pp.rows + (row * kPlanRowsK + (lane & 31)) * RB, lane);
  const float* co = pp.coef + row * kPlanRowsK;
  float cl[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    cl[v] = r < kRetainedK ? co[r] : 0.0f;
  }
  const bool hi_half = lane >= 32;
  const float m_aux = hi_half ? co[kAuxRowK] : 0.0f, m_lin = hi_half ? co[kLinRowK] : 0.0f;
  const float kappa = pp.misc[row * 4 + 0], e_neg = hi_half ? pp.misc[row * 4 + 1] : 0.0f;
  const bool recover = pp.flag[row] != 0;

  uint32_t* my_hist = hist[wave];
  uint64_t* my_stage = stage[wave];
  int32_t* my_q = squeue[wave];
  RowState rs{cand + row * (size_t)cap, 0, 0, 0};
  const uint8_t* kbase = k + (size_t)b * N * RB;
  const float* kscb = (DT == kFP8) ? ksc + (size_t)b * N : nullptr;
  const float* knb = pp.knorm + (size_t)b * N;
  const int nseed = pp.seed_count[b];
  const int32_t* sd = pp.seeds + (size_t)b * pp.seed_stride;
  const uint32_t* sbits = pp.seed_bits + (size_t)b * pp.bits_stride;
  TileFetch<DT> tf;

  // ---------------------------------------------------------------- 1. seeds
  {
    const int ntiles = (nseed + KT - 1) / KT;
    if (ntiles > 0) {
      tf.fetch(kbase, kscb, 0, N, tid, sd, nseed);
      tf.commit(ktile[0], kscale_tile[0], tid);
    }
    wait_vmem_all();
    __syncthreads();
    for (int ti = 0; ti < ntiles; ++ti) {
      const int cur = ti & 1;
      const int ts = ti * KT;
      if (rs.nst) {
        rs.cnt = flush_stage(rs.buf, rs.cnt, my_stage, rs.nst, lane);
        rs.nst = 0;
      }
      if (ti + 1 < ntiles) tf.fetch(kbase, kscb, ts + KT, N, tid, sd, nseed);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int s0 = ts + 32 * sb;
        if (s0 < nseed && sd[s0] < vis) {  // seeds ascend: wave-uniform test
          const int si = s0 + (lane & 31);
          const int key = sd[min(si, nseed - 1)];
          Frag<DT> f;
          load_frag_lds<DT>(f, ktile[cur], 32 * sb + (lane & 31), lane);
          float s = combine_swap(query_partial_w<DT>(qa, f, my_w, lane));
          if constexpr (DT == kFP8) s = apply_scales(s, qscale, kscale_tile[cur][32 * sb + (lane & 31)]);
          append_rec(rs, make_record(s, (uint32_t)key), lane < 32 && si < nseed && key < vis, my_stage, my_hist,
                     topk, cap, lane);
        }
      }
      if (ti + 1 < ntiles) tf.commit(ktile[cur ^ 1], kscale_tile[cur ^ 1], tid);
      __syncthreads();
    }
  }
  // tau: the exact K-th seed record (records below it can never be selected)
  if (rs.nst) {
    rs.cnt = flush_stage(rs.buf, rs.cnt, my_stage, rs.nst, lane);
    rs.nst = 0;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  float tau = -INFINITY;
  if (rs.cnt >= topk) {
    const SelectResult sel = select_records_d8(rs.buf, rs.cnt, (uint32_t)topk, my_hist, true, 0, lane);
    rs.cnt = compact_records_d8(rs.buf, rs.cnt, sel, lane);
    rs.thr = min_record(rs.buf, rs.cnt, lane);
    tau = record_score(rs.thr);
  }

  // ---------------------------------------------------------------- 2-3. screen + refine
  // Key tiles stream through a ring of kRing LDS slots (tile ti in slot
  // ti % kRing).  The screen appends surviving keys to the wave's list
  // my_q[0..nq) (one LDS store per survivor); every kRefineEvery tiles all
  // waves rescore their lists together, 32 keys per MFMA batch, with the key
  // fragments read from the ring (the survivors' tiles are still resident:
  // a slot is refilled only kRing tiles later).  Refining in the same tiles
  // keeps the eight waves, which meet at every tile, in step.
  int nq = 0, screened = 0, survived = 0;
  auto refine_round = [&]() {
    for (int p0 = 0; p0 < nq; p0 += 32) {
      const int n = min(32, nq - p0);
      const int key = my_q[p0 + ((lane & 31) < n ? (lane & 31) : 0)];
      const int tk = key / KT, r = key - tk * KT, slot = tk % kRing;
      Frag<DT> f;
      load_frag_lds<DT>(f, ktile[slot], r, lane);
      float s = combine_swap(query_partial_w<DT>(qa, f, my_w, lane));
      if constexpr (DT == kFP8) s = apply_scales(s, qscale, kscale_tile[slot][r]);
      if (rs.nst > KT) {  // the stage holds KT + 32 records: make room for this batch
        rs.cnt = flush_stage(rs.buf, rs.cnt, my_stage, rs.nst, lane);
        rs.nst = 0;
      }
      append_rec(rs, make_record(s, (uint32_t)key), lane < n, my_stage, my_hist, topk, cap, lane);
    }
    nq = 0;
  };
  {
    const int ntiles = (wg_vis + KT - 1) / KT;
    if (ntiles > 0) {
      tf.fetch(kbase, kscb, 0, N, tid, nullptr, 0, knb, sbits);
      tf.commit(ktile[0], kscale_tile[0], tid, knorm_tile[0], sbits_tile[0]);
    }
    wait_vmem_all();
    __syncthreads();
    const int lk = lane & 31;
    for (int ti = 0; ti < ntiles; ++ti) {
      const int cur = ti % kRing;
      const int ts = ti * KT;
      // The loop is bound by the latency of the next tile's fetch: issue it
      // first, so that refine rounds and cuts run in its shadow.
      if (ti + 1 < ntiles) tf.fetch(kbase, kscb, ts + KT, N, tid, nullptr, 0, knb, sbits);
      if (ti > 0 && ti % kRefineEvery == 0) refine_round();
      if (rs.nst) {
        rs.cnt = flush_stage(rs.buf, rs.cnt, my_stage, rs.nst, lane);
        rs.nst = 0;
      }
      // Keep the survivor threshold near the K-th best exact record seen so
      // far: cut back to exactly topk records whenever kCutSlack more have
      // been kept.
      if (rs.cnt >= topk + kCutSlack) {
        const Cut c = cut_candidates_d8(rs.buf, rs.cnt, my_stage, 0, my_hist, topk, topk, lane);
        rs.cnt = c.cnt;
        rs.thr = c.thr;
      }
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int kb = ts + 32 * sb;
        if (kb < vis) {  // wave-uniform
          // -- bound of 32 keys: one 32x32 block (32 plan rows x 32 keys);
          //    each lane sums its 16 rows, the cross-half exchange the rest
          Frag<DT> kf;
          load_frag_lds<DT>(kf, ktile[cur], 32 * sb + lk, lane);
          const f32x16 dd = mma_block<DT>(sa, kf, zero16());
          const float kn = knorm_tile[cur][32 * sb + lk];
          float p = 0.0f;
#pragma unroll
          for (int v = 0; v < 16; ++v) p = __builtin_fmaf(__builtin_fabsf(dd[v]), cl[v], p);
          p += __builtin_fmaf(m_lin, dd[15], -relu_bits(__builtin_fmaf(m_aux, dd[14], -e_neg * kn)));
          float U = __builtin_fmaf(kappa, kn, combine_swap(p));
          if constexpr (DT == kFP8) U = apply_scales(U, qscale, kscale_tile[cur][32 * sb + lk]);
          const int key = kb + lk;
          const uint32_t seedw = sbits_tile[cur][sb];
          const bool ck = (lane < 32) & (key < vis) & !((seedw >> lk) & 1u);
          const bool sv = ck & (recover | (make_record(U, (uint32_t)key) >= rs.thr));
          if (pp.st_ub && ck) pp.st_ub[row * (size_t)N + key] = U;
          screened += __popcll(__ballot(ck));
          const uint32_t mask = (uint32_t)__ballot(sv);  // bit i: key kb + i survives
          survived += __popc(mask);
          if (mask) {  // append the survivors to the list (key order)
            if (sv) my_q[nq + __popc(mask & ((1u << lk) - 1u))] = key;
            nq += __popc(mask);
          }
        }
      }
      if (ti + 1 < ntiles)
        tf.commit(ktile[(ti + 1) % kRing], kscale_tile[(ti + 1) % kRing], tid, knorm_tile[(ti + 1) % kRing],
                  sbits_tile[(ti + 1) % kRing]);
      __syncthreads();
    }
    refine_round();  // the last tiles' survivors (their slots are untouched)
  }

  // ---------------------------------------------------------------- 4. select
  if (!valid) return;
  emit_topk_d8(rs.buf, rs.cnt, my_stage, rs.nst, my_hist, topk, out_idx + row * (size_t)topk,
            out_score ? out_score + row * (size_t)topk : nullptr, lane);
  if (lane == 0) {
    if (pp.st_tau) pp.st_tau[row] = tau;
    if (pp.st_screened) pp.st_screened[row] = screened;
    if (pp.st_surv) pp.st_surv[row] = survived;
    if (pp.st_rec) pp.st_rec[row] = recover ? 1 : 0;
  }
}

__global__ void k_fill_nan(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = __builtin_nanf("");
}

hipError_t launch_topk_pruned(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx, float* out_score,
                              const PrunedBuffers& pb, hipStream_t st) {
  if (pb.st_ub) {
    const size_t n = (size_t)p.B * p.Q * p.N;
    hipLaunchKernelGGL(k_fill_nan, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pb.st_ub, n);
  }
  PrunePlan pp{pb.plan_rows, pb.plan_coef, pb.plan_misc, pb.plan_flag, pb.knorm, pb.seeds, pb.seed_count,
               pb.seed_stride, pb.seed_bits, pb.bits_stride, pb.st_tau, pb.st_screened, pb.st_surv, pb.st_rec,
               pb.st_ub};
  dim3 grid((p.Q + kWaves - 1) / kWaves, p.B);
  const int prof_slot = prof_open("k_topk_pruned", st);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_topk_pruned<kBF16>, grid, dim3(kWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale,
                       p.pos, p.Q, p.N, topk, cap, cand, out_idx, out_score, pp);
  else
    hipLaunchKernelGGL(k_topk_pruned<kFP8>, grid, dim3(kWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale,
                       p.pos, p.Q, p.N, topk, cap, cand, out_idx, out_score, pp);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

}  // namespace dsa
