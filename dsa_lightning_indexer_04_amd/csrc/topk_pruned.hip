// topk_pruned.hip -- exact Top-K with certified (DoSA) pruning, fused.
//
// Flow per query row (DoSA reading notes, annotation LBKERZAW, steps 1-3;
// 机器之心 DoSA article, sections 03-04, Fig. 2-3):
//   1. seeds: the seed keys are scored with all heads by the same routine as
//      every other path and go into the row's candidate buffer; the K-th best
//      seed record is the threshold tau (K distinct visible keys reach it, so
//      it cannot exceed the true K-th score);
//   2. screen: every other visible key gets the certified upper bound U from
//      32 plan rows (up to 30 retained heads, the folded negative-head row,
//      the linear row; see prune_prep.hip) -- one 32x32 MFMA block per 32
//      keys -- and survives iff U reaches the row's running threshold; a
//      64-lane ballot packs the survivors of a block into a bitmask;
//   3. compact + refine: survivors are queued per row and rescored with all
//      heads in batches of 32 (key rows gathered by index, same score
//      routine), and only records not below the threshold are kept as
//      candidates;
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
// Workgroup geometry per dtype: query rows per workgroup (one per wave), key
// bytes of an LDS tile, tile slots (tiles are loaded kSlots - 1 ahead).  Both
// dtypes use 8 rows on 32 KiB tiles in 3 slots, one workgroup per CU (4 rows
// on 24 KiB tiles in 2 slots, two workgroups per CU, measured no faster on
// fp8 keys: the per-tile work grows with the tile count).
template <int DT>
struct PrunedGeom;
template <>
struct PrunedGeom<kBF16> {
  static constexpr int kWaves = 8, kTileBytes = 32768, kSlots = 3;
};
template <>
struct PrunedGeom<kFP8> {
  static constexpr int kWaves = 8, kTileBytes = 32768, kSlots = 3;
};
constexpr int kStage = 96;       // candidate stage records per row

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
  const int32_t* seed_top_idx;   // [R][topk]: the row's exact seed Top-K (seed numbers, -1 padded)
  const float* seed_top_score;   // [R][topk]: their scores
  float* st_tau;
  int32_t* st_screened;
  int32_t* st_surv;
  uint8_t* st_rec;
  float* st_ub;              // [R][N] debug bounds or null
};

// Keep the records of up to 64 lanes that reach the threshold (stage + one
// histogram count each); a full buffer is compacted first.
__device__ __forceinline__ void append_rec(RowState& rs, uint64_t rec, bool live, uint64_t* stage, uint32_t* hist,
                                           int topk, int cap, int lane) {
  uint64_t bal = __ballot(live && rec >= rs.thr);
  if (bal) {
    if (rs.cnt + rs.nst + __popcll(bal) > cap) {
      apply_rebuild(rs, rebuild_candidates(rs.buf, rs.cnt, stage, rs.nst, hist, rs.thr, topk, cut_goal(topk, cap), lane));
      bal = __ballot(live && rec >= rs.thr);
    }
    if (live && rec >= rs.thr) {
      stage[rs.nst + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] =
          rec;
      atomicAdd(&hist[thr_bin((uint32_t)(rec >> 32), rs.base, rs.shift)], 1u);
    }
    rs.nst += __popcll(bal);
    rs.added += __popcll(bal);
  }
}

// kBounds: also write every screened key's bound U to pp.st_ub (diagnostics).
template <int DT, bool kBounds>
__global__ __launch_bounds__(PrunedGeom<DT>::kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_topk_pruned(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ qsc, const float* __restrict__ ksc, const int32_t* __restrict__ pos, int Q, int N,
    int topk, int cap, uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_score,
    PrunePlan pp) {
  constexpr int kWaves = PrunedGeom<DT>::kWaves, kTileBytes = PrunedGeom<DT>::kTileBytes;
  constexpr int kSlots = PrunedGeom<DT>::kSlots, kAhead = kSlots - 1;  // tiles loaded ahead
  using Tile = DirectTile<DT, kTileBytes, kWaves>;
  constexpr int RB = Frag<DT>::kRowBytes;
  constexpr int KT = Tile::KT;     // keys per tile (128 bf16, 256 fp8)
  constexpr int NSB = KT / 32;     // 32-key blocks per tile (even)
  constexpr int QCAP = KT + 96;    // survivor queue per row (see the refine schedule)
  constexpr int kPend = (DT == kFP8) ? 2 : 1;  // refine batches in flight per tile (register budget)
  __shared__ u32x4 ktile[kSlots][direct_slots(kTileBytes)];
  __shared__ float kscale_tile[kSlots][KT];
  __shared__ float knorm_tile[kSlots][KT];
  __shared__ uint32_t sbits_tile[kSlots][64];
  __shared__ __align__(16) uint32_t hist[kWaves][256];  // radix-select bins (8-bit digits), threshold histogram
  __shared__ uint64_t stage[kWaves][kStage];  // candidate records awaiting a flush
  __shared__ int32_t squeue[kWaves][QCAP + 64];  // survivor keys awaiting refinement (+ scratch)
  __shared__ uint32_t toff[kWaves][Tile::PER_WAVE * 64];
  __shared__ __align__(16) float wrow[kWaves][kHeads];

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
  Frag<DT> qa[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) load_frag<DT>(qa[blk], q + (row * kHeads + 32 * blk + (lane & 31)) * RB, lane);
  wrow[wave][lane] = w[row * kHeads + lane];
  const float* my_w = wrow[wave];
  const float qscale = (DT == kFP8) ? qsc[row] : 1.0f;

  uint32_t* my_hist = hist[wave];
  uint64_t* my_stage = stage[wave];
  int32_t* my_q = squeue[wave];
  for (int i = lane; i < 256; i += 64) my_hist[i] = 0u;  // threshold histogram (coarse bins until the first cut)
  RowState rs{cand + row * (size_t)cap, 0, 0, 0, 0u, 24, 0};
  const uint8_t* kbase = k + (size_t)b * N * RB;
  const float* kscb = (DT == kFP8) ? ksc + (size_t)b * N : nullptr;
  const float* knb = pp.knorm + (size_t)b * N;
  const int nseed = pp.seed_count[b];
  const int32_t* sd = pp.seeds + (size_t)b * pp.seed_stride;
  const uint32_t* sbits = pp.seed_bits + (size_t)b * pp.bits_stride;
  const int lk = lane & 31;
  Tile tl;
  tl.init(toff[wave], wave, lane);

  // Exact scores of up to 32 keys (lane l % 32: key keys_l, fragment f) go
  // to the candidate buffer if their records reach the threshold.
  auto score_and_keep = [&](const Frag<DT>& f, int key, float ks, bool live) {
    float s = combine_swap(query_partial_w<DT>(qa, f, my_w, lane));
    if constexpr (DT == kFP8) s = apply_scales(s, qscale, ks);
    if (rs.nst > kStage - 32) {
      rs.cnt = flush_stage(rs.buf, rs.cnt, my_stage, rs.nst, lane);
      rs.nst = 0;
    }
    append_rec(rs, make_record(s, (uint32_t)key), live, my_stage, my_hist, topk, cap, lane);
  };

  // ---------------------------------------------------------------- 1. seeds
  // The row's exact seed Top-K, scored beforehand by the streaming Top-K over
  // the packed seed keys (the same score routine, so the same bits), become
  // its first candidate records; tau is the K-th best of them.
  {
    const int32_t* si = pp.seed_top_idx + row * (size_t)topk;
    const float* ss = pp.seed_top_score + row * (size_t)topk;
    int nk = 0;
    for (int i0 = 0; i0 < topk; i0 += 64) {
      const int i = i0 + lane;
      const int32_t idx = i < topk ? si[i] : -1;
      const bool ok = valid && idx >= 0;  // rows past Q keep no records
      const uint64_t bal = __ballot(ok);
      if (ok)
        rs.buf[nk + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] =
            make_record(ss[i], (uint32_t)sd[idx]);
      nk += __popcll(bal);
    }
    rs.cnt = nk;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  float tau = -INFINITY;
  if (rs.cnt >= topk) {
    rs.thr = min_record(rs.buf, rs.cnt, lane);
    tau = record_score(rs.thr);
  }
  apply_rebuild(rs, rebuild_candidates(rs.buf, rs.cnt, my_stage, 0, my_hist, rs.thr, topk, cap, lane));
  rs.added = 0;

  // screen side: the 32 plan rows as one 32x32 MFMA A operand; lane l holds
  // rows 8*(v/4) + 4*(l/32) + v%4 of the result (v = 0..15), with their
  // coefficients in cl[v].  Rows 30 (aux) and 31 (linear) land in lanes
  // 32..63 at v = 14, 15, whose cl is zero; they enter the bound separately.
  Frag<DT> sa;
  load_frag<DT>(sa, pp.rows + (row * kPlanRowsK + (lane & 31)) * RB, lane);
  const float* co = pp.coef + row * kPlanRowsK;
  float cl[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    cl[v] = r < kRetainedK ? co[r] : 0.0f;
  }
  const float m_aux = co[kAuxRowK], m_lin = co[kLinRowK];
  const float kappa = pp.misc[row * 4 + 0], e_neg = pp.misc[row * 4 + 1];
  const bool recover = pp.flag[row] != 0;


  // ---------------------------------------------------------------- 2-3. screen + refine
  // Survivors are pushed to the row's queue my_q[qh, nq).  Refine schedule,
  // per tile: at its start, pop up to kPend full batches of 32 queued
  // survivors and issue the loads of their key rows (global memory; the rows
  // were streamed moments ago, so they come from cache); score them at the
  // tile's end, after the screen of the tile has covered the load latency.  A row whose
  // queue still holds more than 96 keys at the tile's end refines further
  // batches on the spot (rows with very many survivors, e.g. recovered
  // rows), so the next tile's KT survivors always fit.
  int qh = 0, nq = 0, screened = 0, survived = 0;
  float thr_f = record_floor(rs.thr);
  auto batch_keys = [&](int n) { return my_q[qh + (lk < n ? lk : 0)]; };
  auto refine_now = [&](int n) {  // pop n <= 32 keys and rescore them synchronously
    const int key = batch_keys(n);
    Frag<DT> f;
    load_frag<DT>(f, kbase + (size_t)key * RB, lane);
    const float ks = (DT == kFP8) ? kscb[key] : 1.0f;
    qh += n;
    score_and_keep(f, key, ks, lane < n);
  };
  {
    const int ntiles = (wg_vis + KT - 1) / KT;
    const int words = pp.bits_stride;
    for (int ti = 0; ti < min(ntiles, kAhead); ++ti) {
      tl.load(ktile[ti], kbase, ti * KT, N, lane);
      if constexpr (DT == kFP8) tl.load_words(kscale_tile[ti], kscb, ti * KT, N, lane);
      tl.load_words(knorm_tile[ti], knb, ti * KT, N, lane);
      tl.load_bits(sbits_tile[ti], sbits, ti * KT, words, lane);
    }
    wait_vmem_all();
    __syncthreads();
    int cur = 0;
    for (int ti = 0; ti < ntiles; ++ti) {
      const int nxt = cur == kSlots - 1 ? 0 : cur + 1;
      const int spare = cur + kAhead >= kSlots ? cur + kAhead - kSlots : cur + kAhead;  // tile ti + kAhead
      const int ts = ti * KT;
      if (rs.nst) {
        rs.cnt = flush_stage(rs.buf, rs.cnt, my_stage, rs.nst, lane);
        rs.nst = 0;
      }
      // Keep the survivor threshold near the K-th best exact record seen so
      // far (to within one histogram bin), at no buffer traffic.
      if (rs.added >= kRaiseEvery) {
        raise_threshold(rs, my_hist, topk, lane);
        thr_f = record_floor(rs.thr);
      }
      if (ti + kAhead < ntiles) {
        const int tn = (ti + kAhead) * KT;
        tl.load(ktile[spare], kbase, tn, N, lane);
        if constexpr (DT == kFP8) tl.load_words(kscale_tile[spare], kscb, tn, N, lane);
        tl.load_words(knorm_tile[spare], knb, tn, N, lane);
        tl.load_bits(sbits_tile[spare], sbits, tn, words, lane);
      }
      // refine batches, part 1: pop up to kPend full batches and issue the
      // loads of their key rows
      const int npend = min(kPend, (nq - qh) >> 5);
      Frag<DT> rf[kPend];
      int rkey[kPend];
      float rks[kPend];
#pragma unroll
      for (int i = 0; i < kPend; ++i) {
        rkey[i] = 0;
        rks[i] = 1.0f;
        if (i < npend) {
          rkey[i] = batch_keys(32);
          load_frag<DT>(rf[i], kbase + (size_t)rkey[i] * RB, lane);
          if constexpr (DT == kFP8) rks[i] = kscb[rkey[i]];
          qh += 32;
        }
      }
      // screen, two 32-key blocks (64 keys, one per lane after the exchange)
      // at a time: the 32x32 MFMA block of each (32 plan rows x 32 keys),
      // each lane's 16 retained-row terms in two chains, then one lane swap
      // pairs the two halves of every key's sum -- lane l ends up with key
      // kb + l -- and two more bring the aux and linear rows' dots (rows 30,
      // 31, held by lanes 32..63) to the same layout.
      auto screen_pair = [&](int pr) {
        const int kb = ts + 64 * pr;
        Frag<DT> kf;
        Tile::frag(kf, ktile[cur], 64 * pr + lk, lane);
        const f32x16 dA = mma_block<DT>(sa, kf, zero16());
        Tile::frag(kf, ktile[cur], 64 * pr + 32 + lk, lane);
        const f32x16 dB = mma_block<DT>(sa, kf, zero16());
        float a0 = 0.0f, a1 = 0.0f, b0 = 0.0f, b1 = 0.0f;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          a0 = __builtin_fmaf(__builtin_fabsf(dA[v]), cl[v], a0);
          a1 = __builtin_fmaf(__builtin_fabsf(dA[v + 8]), cl[v + 8], a1);
          b0 = __builtin_fmaf(__builtin_fabsf(dB[v]), cl[v], b0);
          b1 = __builtin_fmaf(__builtin_fabsf(dB[v + 8]), cl[v + 8], b1);
        }
        float sA = a0 + a1, sB = b0 + b1;
        swap_halves(sA, sB);
        float xA = dA[14], xB = dB[14], yA = dA[15], yB = dB[15];
        swap_halves(xA, xB);  // xB: row-30 (aux) dot of key kb + lane
        swap_halves(yA, yB);  // yB: row-31 (linear) dot of key kb + lane
        const float kn = knorm_tile[cur][64 * pr + lane];
        float U = __builtin_fmaf(m_lin, yB, sA + sB);
        U -= relu_bits(__builtin_fmaf(m_aux, xB, -e_neg * kn));
        U = __builtin_fmaf(kappa, kn, U);
        if constexpr (DT == kFP8) U = apply_scales(U, qscale, kscale_tile[cur][64 * pr + lane]);
        const int key = kb + lane;
        const uint32_t seedw = sbits_tile[cur][2 * pr + (lane >> 5)];
        const bool ck = (key < vis) & !((seedw >> lk) & 1u);
        // U >= the threshold's float floor keeps every key whose record
        // (U, key) reaches the threshold (and at most a few equal-bound keys
        // below it, which the refine drops)
        const bool sv = ck & (recover | (U >= thr_f));
        if constexpr (kBounds) {
          if (ck) pp.st_ub[row * (size_t)N + key] = U;
        }
        screened += __popcll(__ballot(ck));
        const uint64_t mask = __ballot(sv);  // bit l: key kb + l survives
        const int before =
            (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        my_q[sv ? nq + before : QCAP + lane] = key;  // branch-free: the others write scratch slots
        nq += __popcll(mask);
        survived += __popcll(mask);
      };
      if (ts + KT <= vis) {  // a whole visible tile: one straight run of pairs
#pragma unroll
        for (int pr = 0; pr < NSB / 2; ++pr) screen_pair(pr);
      } else {
#pragma unroll
        for (int pr = 0; pr < NSB / 2; ++pr)
          if (ts + 64 * pr < vis) screen_pair(pr);  // wave-uniform
      }
      // refine batches, part 2: score the popped keys
#pragma unroll
      for (int i = 0; i < kPend; ++i)
        if (i < npend) score_and_keep(rf[i], rkey[i], rks[i], lane < 32);
      // compact the queue to its front; refine on the spot while it is long
      if (qh > 0) {
        const int left = nq - qh;
        for (int i = lane; i < left; i += 64) {
          const int v = my_q[qh + i];
          __builtin_amdgcn_wave_barrier();
          my_q[i] = v;
        }
        nq = left;
        qh = 0;
      }
      while (nq > QCAP - KT) {
        refine_now(32);
        const int left = nq - qh;
        for (int i = lane; i < left; i += 64) {
          const int v = my_q[qh + i];
          __builtin_amdgcn_wave_barrier();
          my_q[i] = v;
        }
        nq = left;
        qh = 0;
      }
      thr_f = record_floor(rs.thr);
      wait_vmem_all();
      __syncthreads();
      cur = nxt;
    }
    while (nq > qh) refine_now(min(32, nq - qh));  // the last survivors
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

#define DSA_PRUNED_KERNEL(DT_, B_)                                                                             \
  template __global__ void k_topk_pruned<DT_, B_>(const uint8_t* __restrict__, const uint8_t* __restrict__,   \
                                                  const float* __restrict__, const float* __restrict__,       \
                                                  const float* __restrict__, const int32_t* __restrict__, int, \
                                                  int, int, int, uint64_t* __restrict__, int32_t* __restrict__, \
                                                  float* __restrict__, PrunePlan);
DSA_PRUNED_KERNEL(kBF16, false)
DSA_PRUNED_KERNEL(kBF16, true)
DSA_PRUNED_KERNEL(kFP8, false)
DSA_PRUNED_KERNEL(kFP8, true)
#undef DSA_PRUNED_KERNEL

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
  PrunePlan pp{pb.plan_rows,    pb.plan_coef,    pb.plan_misc,      pb.plan_flag,    pb.knorm,
               pb.seeds,        pb.seed_count,   pb.seed_stride,    pb.seed_bits,    pb.bits_stride,
               pb.seed_top_idx, pb.seed_top_score, pb.st_tau,       pb.st_screened,  pb.st_surv,
               pb.st_rec,       pb.st_ub};
  const int waves = p.dtype == kBF16 ? PrunedGeom<kBF16>::kWaves : PrunedGeom<kFP8>::kWaves;
  dim3 grid((p.Q + waves - 1) / waves, p.B);
  const int prof_slot = prof_open("k_topk_pruned", st);
  using Kern = void (*)(const uint8_t*, const uint8_t*, const float*, const float*, const float*, const int32_t*, int,
                        int, int, int, uint64_t*, int32_t*, float*, PrunePlan);
  const Kern kern = p.dtype == kBF16 ? (pb.st_ub ? k_topk_pruned<kBF16, true> : k_topk_pruned<kBF16, false>)
                                     : (pb.st_ub ? k_topk_pruned<kFP8, true> : k_topk_pruned<kFP8, false>);
  hipLaunchKernelGGL(kern, grid, dim3(waves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos, p.Q, p.N, topk,
                     cap, cand, out_idx, out_score, pp);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

}  // namespace dsa
