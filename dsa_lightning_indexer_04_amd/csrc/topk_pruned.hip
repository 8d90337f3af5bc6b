// topk_pruned.hip -- exact Top-K with certified (DoSA) pruning, in key chunks.
//
// Flow per query row (DoSA reading notes, annotation LBKERZAW, steps 1-3;
// 机器之心 DoSA article, sections 03-04, Fig. 2-3):
//   1. seeds: the seed keys are scored with all heads by the same routine as
//      every other path (the streaming Top-K over the packed seeds); the
//      row's exact seed Top-K become its first candidate records and the
//      K-th of them is the threshold tau (K distinct visible keys reach it,
//      so it cannot exceed the true K-th score);
//   2. screen: every other visible key of a key chunk gets the certified
//      upper bound U from 32 plan rows (up to 30 retained heads, the folded
//      negative-head row, the linear row; see prune_prep.hip) -- one 32x32
//      MFMA block per 32 keys -- and survives iff U reaches the row's
//      running threshold; a 64-lane ballot packs the survivors of 64 keys
//      into one bitmask word, written to the workspace;
//   3. compact + refine: the row's bitmask words are expanded into survivor
//      key lists (popcount prefix sums) and the survivors are rescored with
//      all heads in batches of 32 (key rows gathered by index, same score
//      routine); records not below the threshold are kept as candidates,
//      and the threshold rises to within one histogram bin of the K-th best
//      exact record seen;
//   4. select: after the last chunk the row's candidates (seed Top-K and
//      refined survivors) are cut to the exact Top-K by score, then key index.
// Keys are taken in chunks of growing length (the first ones short), each
// chunk screened with the threshold the previous chunks' refinement left,
// so most keys meet a threshold close to the row's final K-th score.  The
// bounds never rank: only exact scores do.
// Work split (gfx950): the screen shares each LDS key tile among 8 rows, two
// per wave, so one key fragment read feeds two rows' MFMA blocks; the refine
// runs one wave per row with no barriers, so rows with many survivors delay
// only themselves.
// Recovery: rows flagged by the planner (non-finite plan, forced, invalid
// seeds) are skipped by the screen and refine and recomputed afterwards by
// the unpruned streaming Top-K.
#include <math.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "kernels.h"
#include "stream_common.h"

namespace dsa {

constexpr int kPlanRowsK = 32;
constexpr int kLinRowK = 31;
constexpr int kAuxRowK = 30;
constexpr int kRetainedK = 30;
constexpr int kStage = 96;           // candidate stage records per row (refine)
constexpr int kScreenWaves = 4;      // screen: waves per workgroup, two rows each
constexpr int kScreenTile = 16384;   // screen: key bytes of an LDS tile
constexpr int kScreenSlots = 3;      // screen: tile slots (two tiles loaded ahead)
constexpr int kRefineWaves = 4;      // refine: rows per workgroup, one per wave
constexpr int kGroupWords = 64;      // refine: bitmask words expanded at a time (one per lane)
constexpr int kQueue = 64 * kGroupWords + 64;  // refine: survivor queue per row

static_assert(sizeof(PruneRowCtl) == 64, "row control block layout");

struct PruneArgs {
  const uint8_t* rows;       // [R][32][128] dtype: bound rows
  const float* coef;         // [R][32]: c_0..c_29, aux multiplier, linear multiplier
  const float* misc;         // [R][4]: kappa, e_neg
  int32_t* flag;             // [R]: 1 = recover (no pruning); the final refine sets it on a raised-start miss
  const float* knorm;        // [B][N]: |k|, rounded up
  const int32_t* seeds;      // [B][seed_stride] ascending
  int seed_stride;
  const uint32_t* seed_bits; // [B][bits_stride]
  int bits_stride;
  const int32_t* seed_pos;       // [R]: the row's visible seeds - 1
  int raised_start;
  int compact;                   // 32-bit candidate records
  const int32_t* seed_top_idx;   // [R][topk]: the row's exact seed Top-K (seed numbers, -1 padded)
  const float* seed_top_score;   // [R][topk]: their scores
  PruneRowCtl* ctl;          // [R]
  uint32_t* hist;            // [R][256]: threshold histogram between launches
  uint64_t* mask;            // [R][mask_stride]: survivor bitmask of the current chunk
  int mask_stride;
  float* st_tau;
  int32_t* st_screened;
  int32_t* st_surv;
  uint8_t* st_rec;
  float* st_ub;              // [R][N] debug bounds or null
};

// ---------------------------------------------------------------- 1. seeds

// ---------------------------------------------------------------- compact records

// Key index bits of a compact record for N keys.
__device__ __forceinline__ int key_bits(int N) { return N <= 2 ? 1 : 32 - __builtin_clz((uint32_t)(N - 1)); }

// A row's compact 32-bit record (DoSA reading notes, annotation TMIF4XYF:
// a compact monotone score code plus the exact key index): the low kb bits
// hold 2^kb - 1 - key, the high 32 - kb bits the code
//   c(m) = min(2^(32-kb) - 1, (m - cbase) >> cshift)
// of the score's monotone code m, for m >= cbase (the row's start; records
// below the start are never kept).  c is monotone in the score: records of
// different codes are ordered by score, records of one code are not.
struct Code32 {
  uint32_t cbase;
  int cshift, kb;
  __device__ __forceinline__ uint32_t cmax() const { return 0xFFFFFFFFu >> kb; }
  __device__ __forceinline__ uint32_t kmask() const { return (1u << kb) - 1u; }
  __device__ __forceinline__ uint32_t code(uint32_t m) const {
    return m <= cbase ? 0u : min(cmax(), (m - cbase) >> cshift);
  }
  __device__ __forceinline__ uint32_t make(uint64_t rec) const {
    return (code((uint32_t)(rec >> 32)) << kb) | (kmask() - record_key(rec));
  }
  __device__ __forceinline__ uint32_t key(uint32_t r) const { return kmask() - (r & kmask()); }
  // The 64-bit threshold record of code c >= 1: every record whose code is
  // at least c is at least this (the lower edge of code c).
  __device__ __forceinline__ uint64_t edge(uint32_t c) const {
    const uint64_t m = (uint64_t)cbase + ((uint64_t)c << cshift);
    return (m > 0xFFFFFFFFull ? 0xFFFFFFFFull : m) << 32;
  }
};

// Candidate state of one row with compact records (wave-uniform).  thr is
// the 64-bit threshold record (the start, or the lower edge of code cthr):
// a record is kept iff it reaches thr, so every kept record reaches the
// start.  The threshold histogram counts kept codes, bin
// min(255, (c - hbase) >> hshift), hbase <= cthr.  dead: a cut could not
// make room (one code holds too many records); the row is recomputed.
struct RowState32 {
  uint32_t* buf;
  int cnt, nst;
  uint64_t thr;
  uint32_t cthr, hbase;
  int hshift, added;
  bool dead;
};

// In place, in order: keep the records whose code is at least cmin.
static __device__ __noinline__ int compact32(uint32_t* buf, int cnt, uint32_t cmin, int kb, int lane) {
  int base = 0;
  for (int i0 = 0; i0 < cnt; i0 += 512) {
    uint32_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      r[j] = i < cnt ? buf[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      const bool keep = i < cnt && (r[j] >> kb) >= cmin;
      const uint64_t bal = __ballot(keep);
      if (keep) buf[base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = r[j];
      base += __popcll(bal);
    }
  }
  return base;
}

// Radix selection over the codes of cnt records (1 <= need <= cnt): digits
// of at most 8 code bits from the top.  Returns a code-aligned threshold
// cmin with `above` records in higher digit groups and `at` in cmin's group
// (above < need <= above + at).  It stops once the boundary group is taken
// whole (above + at == need), or, given a goal, once above + at <= goal;
// otherwise every code bit is fixed and cmin's group is the single code
// cmin.
struct CodeCut {
  uint32_t cmin, above, at;
};
static __device__ __noinline__ CodeCut select_code32(const uint32_t* buf, int cnt, uint32_t need, int kb,
                                                      uint32_t* hist, uint32_t goal, int lane) {
  const int cb = 32 - kb;
  uint32_t prefix = 0, remaining = need, above = 0, at = (uint32_t)cnt;
  int done = 0;
  while (done < cb) {
    const int width = min(8, cb - done);
    const int lo = kb + cb - done - width;  // lowest record bit of this digit
    const int hi = lo + width;              // record bits from here up hold the fixed prefix
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = lane; i < 256; i += 64) hist[i] = 0u;
    wave_lds_sync();
    for (int i0 = 0; i0 < cnt; i0 += 512) {
      uint32_t r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + 64 * j + lane;
        r[j] = i < cnt ? buf[i] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = i0 + 64 * j + lane;
        const uint32_t top = hi >= 32 ? 0u : r[j] >> hi;
        if (i < cnt && top == prefix) atomicAdd(&hist[(r[j] >> lo) & dmask], 1u);
      }
    }
    wave_lds_sync();
    uint32_t bin, ab, count;
    find_boundary(hist, 256, remaining, lane, bin, ab, count);
    prefix = (prefix << width) | bin;
    above += ab;
    remaining -= ab;
    at = count;
    done += width;
    if (count == remaining) break;
    if (goal && above + count <= goal) break;
  }
  return {prefix << (cb - done), above, at};
}

// Flush the stage; keep the records of codes >= cthr; if more than `goal`
// remain, cut to the codes of the best topk (whole codes: the threshold
// becomes the boundary code's lower edge); mark the row dead when the cut
// leaves no room for two more stages; refit the histogram.  (Arguments and
// result by value: a reference to the caller's row state would put that
// state in scratch memory for the whole refine loop.)
struct Rebuilt32 {
  int cnt;
  uint64_t thr;
  uint32_t cthr, hbase;
  int hshift;
  bool dead;
};
static __device__ __noinline__ Rebuilt32 rebuild32(uint32_t* buf, int cnt, const uint32_t* stage, int nst,
                                                   uint32_t* hist, Code32 code, uint64_t thr, uint32_t cthr,
                                                   int topk, int goal, int cap, int lane) {
  for (int i = lane; i < nst; i += 64) buf[cnt + i] = stage[i];
  cnt += nst;
  row_mem_sync();
  cnt = compact32(buf, cnt, cthr, code.kb, lane);
  if (cnt > goal) {
    row_mem_sync();
    const CodeCut cut = select_code32(buf, cnt, (uint32_t)topk, code.kb, hist, (uint32_t)goal, lane);
    if (cut.cmin > cthr) {
      row_mem_sync();
      cnt = compact32(buf, cnt, cut.cmin, code.kb, lane);
      cthr = cut.cmin;
      thr = code.edge(cut.cmin);
    }
  }
  row_mem_sync();
  uint32_t mx = cthr;
  for (int i = lane; i < cnt; i += 64) mx = max(mx, buf[i] >> code.kb);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d, 64));
  const uint32_t span = mx - cthr;
  const int hshift = span ? max(0, 24 - (int)__builtin_clz(span)) : 0;
  for (int i = lane; i < 256; i += 64) hist[i] = 0u;
  wave_lds_sync();
  for (int i = lane; i < cnt; i += 64) atomicAdd(&hist[thr_bin(buf[i] >> code.kb, cthr, hshift)], 1u);
  wave_lds_sync();
  return {cnt, thr, cthr, cthr, hshift, cnt > cap - 4 * kStage};
}

// raise_threshold on the code histogram: the threshold rises to the lower
// edge of the highest code that at least topk kept records reach.
__device__ __forceinline__ void raise32(RowState32& rc, const uint32_t* hist, const Code32& code, int topk, int lane) {
  const u32x4 h = reinterpret_cast<const u32x4*>(hist)[63 - lane];  // h.w: bin 255 - 4 lane
  const uint32_t local = h.x + h.y + h.z + h.w;
  const uint32_t above = wave_prefix_incl(local, lane) - local;
  const uint64_t bal = __ballot(above < (uint32_t)topk && (uint32_t)topk <= above + local);
  rc.added = 0;
  if (!bal) return;
  const int src = __builtin_ctzll(bal);
  uint32_t b = 4u * (63 - lane);
  if (above + h.w >= (uint32_t)topk)
    b += 3;
  else if (above + h.w + h.z >= (uint32_t)topk)
    b += 2;
  else if (above + h.w + h.z + h.y >= (uint32_t)topk)
    b += 1;
  b = (uint32_t)__builtin_amdgcn_readlane((int)b, src);
  const uint32_t c = rc.hbase + (b << rc.hshift);
  if (c > rc.cthr) {
    rc.cthr = c;
    rc.thr = code.edge(c);
  }
}

// append_rec with compact records: the 64-bit record decides (it must
// reach thr), the compact one is stored.
__device__ __forceinline__ void append32(RowState32& rc, uint64_t rec, bool live, uint32_t* stage, uint32_t* hist,
                                         const Code32& code, int topk, int cap, int lane) {
  bool keep = live && !rc.dead && rec >= rc.thr;
  uint64_t bal = __ballot(keep);
  if (bal) {
    if (rc.cnt + rc.nst + __popcll(bal) > cap) {
      const Rebuilt32 rb = rebuild32(rc.buf, rc.cnt, stage, rc.nst, hist, code, rc.thr, rc.cthr, topk,
                                     cut_goal(topk, cap), cap, lane);
      rc.cnt = rb.cnt;
      rc.nst = 0;
      rc.thr = rb.thr;
      rc.cthr = rb.cthr;
      rc.hbase = rb.hbase;
      rc.hshift = rb.hshift;
      rc.added = kRaiseEvery;
      rc.dead = rc.dead || rb.dead;
      keep = live && !rc.dead && rec >= rc.thr;
      bal = __ballot(keep);
    }
    if (keep) {
      const uint32_t r = code.make(rec);
      stage[rc.nst + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = r;
      atomicAdd(&hist[thr_bin(r >> code.kb, rc.hbase, rc.hshift)], 1u);
    }
    rc.nst += __popcll(bal);
    rc.added += __popcll(bal);
  }
}

// Seed rank of a row's raised start: with S seeds spread evenly over the
// row's V visible keys, the number of seeds at or above the K-th score is
// about mu = K S / V (a binomial count when the scores do not depend on the
// position), so the m-th best seed, m = ceil(mu + 5 sqrt(mu)) + 1, is a
// score that at least K keys reach unless the count falls five standard
// deviations short.  m >= K means no raise.
__device__ __forceinline__ int raised_start_rank(int topk, int seeds, int vis) {
  if (seeds <= 0 || vis <= 0) return topk;
  const float mu = (float)topk * (float)seeds / (float)vis;
  if (mu >= (float)topk) return topk;
  return (int)ceilf(mu + 5.0f * sqrtf(mu)) + 1;
}

// One wave per row: the row's seed Top-K records into its candidate buffer,
// tau = the K-th of them.  The running threshold starts at tau, or (raised
// start) at the record of seed rank raised_start_rank, and the buffer keeps
// the seed records that reach it; the threshold histogram is fitted to them
// and the row's state goes to its control block.  Compact records: the row's
// code is fitted (cbase = the start's code; cshift so that twice the span
// from the start to the best seed fits the code bits) and the kept seed
// records are rewritten as compact records into the second half of the
// row's buffer (the first half is the scratch of the final rescoring).
__global__ __launch_bounds__(kRefineWaves * 64) void k_prune_init(const int32_t* __restrict__ pos, int Q, int N,
                                                                  size_t R, int topk, int cap,
                                                                  uint64_t* __restrict__ cand, PruneArgs pa) {
  __shared__ __align__(16) uint32_t hist[kRefineWaves][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * kRefineWaves + wave;
  if (row >= R) return;  // whole wave; the waves share nothing
  const int b = (int)(row / (size_t)Q);
  uint32_t* my_hist = hist[wave];
  for (int i = lane; i < 256; i += 64) my_hist[i] = 0u;
  RowState rs{cand + row * (size_t)cap, 0, 0, 0, 0u, 24, 0};
  const int32_t* si = pa.seed_top_idx + row * (size_t)topk;
  const float* ss = pa.seed_top_score + row * (size_t)topk;
  const int32_t* sd = pa.seeds + (size_t)b * pa.seed_stride;
  int nk = 0;
  for (int i0 = 0; i0 < topk; i0 += 64) {
    const int i = i0 + lane;
    const int32_t idx = i < topk ? si[i] : -1;
    const bool ok = idx >= 0;
    const uint64_t bal = __ballot(ok);
    if (ok)
      rs.buf[nk + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] =
          make_record(ss[i], (uint32_t)sd[idx]);
    nk += __popcll(bal);
  }
  rs.cnt = nk;
  row_mem_sync();
  float tau = -INFINITY;
  int raised = 0;
  if (rs.cnt >= topk) {
    rs.thr = min_record(rs.buf, rs.cnt, lane);
    tau = record_score(rs.thr);
    const int vis = min(max(pos[row] + 1, 0), N);
    const int m = pa.raised_start && !pa.flag[row] ? raised_start_rank(topk, pa.seed_pos[row] + 1, vis) : topk;
    if (m < topk) {  // the m best records: exactly those at or above the selection's prefix
      rs.thr = select_records_d8(rs.buf, rs.cnt, (uint32_t)m, my_hist, true, 0, lane).prefix;
      raised = 1;
    }
  }
  apply_rebuild(rs, rebuild_candidates(rs.buf, rs.cnt, nullptr, 0, my_hist, rs.thr, topk, cap, lane));
  row_mem_sync();
  uint32_t cbase = 0;
  int cshift = 0;
  if (pa.compact) {
    cbase = (uint32_t)(rs.thr >> 32);
    uint32_t top = cbase;
    for (int i = lane; i < rs.cnt; i += 64) top = max(top, (uint32_t)(rs.buf[i] >> 32));
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) top = max(top, (uint32_t)__shfl_xor((int)top, d, 64));
    const int kb = key_bits(N);
    const uint64_t span2 = 2ull * (uint64_t)(top - cbase);
    cshift = span2 ? max(0, (64 - (int)__builtin_clzll(span2)) - (32 - kb)) : 0;
    const Code32 code{cbase, cshift, kb};
    uint32_t* b32 = reinterpret_cast<uint32_t*>(rs.buf) + cap;
    uint32_t mx = 0;
    for (int i = lane; i < rs.cnt; i += 64) {
      const uint32_t r = code.make(rs.buf[i]);
      b32[i] = r;
      mx = max(mx, r >> kb);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d, 64));
    // the code histogram from code 0 (the start)
    rs.base = 0u;
    rs.shift = mx ? max(0, 24 - (int)__builtin_clz(mx)) : 0;
    for (int i = lane; i < 256; i += 64) my_hist[i] = 0u;
    wave_lds_sync();
    for (int i = lane; i < rs.cnt; i += 64) atomicAdd(&my_hist[thr_bin(b32[i] >> kb, 0u, rs.shift)], 1u);
    wave_lds_sync();
    row_mem_sync();
  }
  uint32_t* gh = pa.hist + row * 256;
  for (int i = lane; i < 256; i += 64) gh[i] = my_hist[i];
  if (lane == 0)
    pa.ctl[row] = PruneRowCtl{rs.thr, rs.cnt, rs.base, rs.shift, 0, 0, 0, tau, raised, cbase, cshift, 0, {0, 0, 0}};
}

// ---------------------------------------------------------------- 2. screen

// The screen side of one row: its 32 plan rows as one 32x32 MFMA A operand
// and the bound's coefficients.  Lane l holds rows 8*(v/4) + 4*(l/32) + v%4
// of a result block (v = 0..15), with their coefficients in cl[v]; rows 30
// (aux) and 31 (linear) land in lanes 32..63 at v = 14, 15, whose cl is
// zero: they enter the bound separately.
template <int DT>
struct ScreenRow {
  Frag<DT> a;
  float cl[16];
  float m_aux, m_lin, kappa, e_neg, qscale, thr_f;
  int vis;
};

template <int DT>
__device__ __forceinline__ void load_screen_row(ScreenRow<DT>& sr, const PruneArgs& pa, const float* qsc, size_t row,
                                                int vis, int lane) {
  constexpr int RB = Frag<DT>::kRowBytes;
  load_frag<DT>(sr.a, pa.rows + (row * kPlanRowsK + (lane & 31)) * RB, lane);
  const float* co = pa.coef + row * kPlanRowsK;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    sr.cl[v] = r < kRetainedK ? co[r] : 0.0f;
  }
  sr.m_aux = co[kAuxRowK];
  sr.m_lin = co[kLinRowK];
  sr.kappa = pa.misc[row * 4 + 0];
  sr.e_neg = pa.misc[row * 4 + 1];
  sr.qscale = (DT == kFP8) ? qsc[row] : 1.0f;
  sr.thr_f = record_floor(pa.ctl[row].thr);
  sr.vis = vis;
}

// The bound of the 64 keys of two 32-key blocks (dA: keys kb..kb+31, dB:
// kb+32..kb+63) for one row; lane l gets key kb + l.  Each lane's 16
// retained-row terms in two chains per block, then one lane swap pairs the
// two halves of every key's sum, and two more bring the aux and linear rows'
// dots (rows 30, 31, held by lanes 32..63) to the same layout.
template <int DT>
__device__ __forceinline__ float pair_bound(const ScreenRow<DT>& sr, const f32x16& dA, const f32x16& dB, float kn,
                                            float ks) {
  float a0 = 0.0f, a1 = 0.0f, b0 = 0.0f, b1 = 0.0f;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    a0 = __builtin_fmaf(__builtin_fabsf(dA[v]), sr.cl[v], a0);
    a1 = __builtin_fmaf(__builtin_fabsf(dA[v + 8]), sr.cl[v + 8], a1);
    b0 = __builtin_fmaf(__builtin_fabsf(dB[v]), sr.cl[v], b0);
    b1 = __builtin_fmaf(__builtin_fabsf(dB[v + 8]), sr.cl[v + 8], b1);
  }
  float sA = a0 + a1, sB = b0 + b1;
  swap_halves(sA, sB);
  float xA = dA[14], xB = dB[14], yA = dA[15], yB = dB[15];
  swap_halves(xA, xB);  // xB: row-30 (aux) dot of key kb + lane
  swap_halves(yA, yB);  // yB: row-31 (linear) dot of key kb + lane
  float U = __builtin_fmaf(sr.m_lin, yB, sA + sB);
  U -= relu_bits(__builtin_fmaf(sr.m_aux, xB, -sr.e_neg * kn));
  U = __builtin_fmaf(sr.kappa, kn, U);
  if constexpr (DT == kFP8) U = apply_scales(U, sr.qscale, ks);
  return U;
}

// Screen of keys [k0, k1): 2 * kScreenWaves rows per workgroup (rows 2w and
// 2w + 1 of the group in wave w) share each key tile; word (s - k0) / 64 of
// a row's bitmask holds the survivors among keys s..s+63 (bit l: key s + l).
// Words past the row's visible prefix are written as zero up to the end of
// the workgroup's last tile; the refine reads only the words below the
// row's prefix.  kBounds: also write every screened key's bound U to
// pa.st_ub (diagnostics).
template <int DT, bool kBounds>
__global__ __launch_bounds__(kScreenWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_screen(
    const float* __restrict__ qsc, const uint8_t* __restrict__ k, const float* __restrict__ ksc,
    const int32_t* __restrict__ pos, int Q, int N, int k0, int k1, PruneArgs pa) {
  using Tile = DirectTile<DT, kScreenTile, kScreenWaves>;
  constexpr int RB = Frag<DT>::kRowBytes;
  constexpr int KT = Tile::KT;     // keys per tile (64 bf16, 128 fp8)
  constexpr int NP = KT / 64;      // 64-key pairs (bitmask words) per tile
  constexpr int kAhead = kScreenSlots - 1;
  __shared__ u32x4 ktile[kScreenSlots][direct_slots(kScreenTile)];
  __shared__ float kscale_tile[kScreenSlots][KT];
  __shared__ float knorm_tile[kScreenSlots][KT];
  __shared__ uint32_t sbits_tile[kScreenSlots][64];
  __shared__ uint32_t toff[kScreenWaves][Tile::PER_WAVE * 64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int group = gridDim.x - 1 - blockIdx.x;  // longest prefixes first
  const int b = blockIdx.y;
  constexpr int kRows = 2 * kScreenWaves;
  // a row takes part if it exists and is not flagged for recovery
  auto row_vis = [&](int t) {
    if (t >= Q) return 0;
    const size_t r = (size_t)b * Q + t;
    return pa.flag[r] ? 0 : min(max(pos[r] + 1, 0), N);
  };
  int wg_end = k0;
  for (int j = 0; j < kRows; ++j) wg_end = max(wg_end, min(k1, row_vis(group * kRows + j)));
  const int t0 = group * kRows + 2 * wave;
  const bool valid0 = t0 < Q, valid1 = t0 + 1 < Q;
  const size_t row0 = (size_t)b * Q + min(t0, Q - 1), row1 = (size_t)b * Q + min(t0 + 1, Q - 1);
  ScreenRow<DT> r0, r1;
  load_screen_row<DT>(r0, pa, qsc, row0, row_vis(t0), lane);
  load_screen_row<DT>(r1, pa, qsc, row1, row_vis(t0 + 1), lane);
  uint64_t* mrow0 = pa.mask + row0 * (size_t)pa.mask_stride;
  uint64_t* mrow1 = pa.mask + row1 * (size_t)pa.mask_stride;

  const uint8_t* kbase = k + (size_t)b * N * RB;
  const float* kscb = (DT == kFP8) ? ksc + (size_t)b * N : nullptr;
  const float* knb = pa.knorm + (size_t)b * N;
  const uint32_t* sbits = pa.seed_bits + (size_t)b * pa.bits_stride;
  const int words = pa.bits_stride;
  const int lk = lane & 31;
  Tile tl;
  tl.init(toff[wave], wave, lane);
  const int ntiles = (wg_end - k0 + KT - 1) / KT;
  for (int ti = 0; ti < min(ntiles, kAhead); ++ti) {
    const int ts = k0 + ti * KT;
    tl.load(ktile[ti], kbase, ts, N, lane);
    if constexpr (DT == kFP8) tl.load_words(kscale_tile[ti], kscb, ts, N, lane);
    tl.load_words(knorm_tile[ti], knb, ts, N, lane);
    tl.load_bits(sbits_tile[ti], sbits, ts, words, lane);
  }
  wait_vmem_all();
  __syncthreads();

  int screened0 = 0, screened1 = 0, survived0 = 0, survived1 = 0;
  // bitmask words of the previous tile, lane j holding pair j; written at
  // the start of the next tile so that the stores complete under its work
  uint64_t pend0 = 0, pend1 = 0;
  int pend_w = -1;
  auto flush_words = [&]() {
    if (pend_w >= 0 && lane < NP) {
      if (valid0) mrow0[pend_w + lane] = pend0;
      if (valid1) mrow1[pend_w + lane] = pend1;
    }
  };
  int cur = 0;
  for (int ti = 0; ti < ntiles; ++ti) {
    const int nxt = cur == kScreenSlots - 1 ? 0 : cur + 1;
    const int spare = cur + kAhead >= kScreenSlots ? cur + kAhead - kScreenSlots : cur + kAhead;
    const int ts = k0 + ti * KT;
    if (ti + kAhead < ntiles) {
      const int tn = ts + kAhead * KT;
      tl.load(ktile[spare], kbase, tn, N, lane);
      if constexpr (DT == kFP8) tl.load_words(kscale_tile[spare], kscb, tn, N, lane);
      tl.load_words(knorm_tile[spare], knb, tn, N, lane);
      tl.load_bits(sbits_tile[spare], sbits, tn, words, lane);
    }
    flush_words();
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      Frag<DT> kfA, kfB;
      Tile::frag(kfA, ktile[cur], 64 * pr + lk, lane);
      Tile::frag(kfB, ktile[cur], 64 * pr + 32 + lk, lane);
      const f32x16 dA0 = mma_block<DT>(r0.a, kfA, zero16());
      const f32x16 dB0 = mma_block<DT>(r0.a, kfB, zero16());
      const f32x16 dA1 = mma_block<DT>(r1.a, kfA, zero16());
      const f32x16 dB1 = mma_block<DT>(r1.a, kfB, zero16());
      const float kn = knorm_tile[cur][64 * pr + lane];
      const float ks = (DT == kFP8) ? kscale_tile[cur][64 * pr + lane] : 1.0f;
      const float U0 = pair_bound<DT>(r0, dA0, dB0, kn, ks);
      const float U1 = pair_bound<DT>(r1, dA1, dB1, kn, ks);
      const int key = ts + 64 * pr + lane;
      const uint32_t seedw = sbits_tile[cur][2 * pr + (lane >> 5)];
      const bool notseed = !((seedw >> lk) & 1u);
      const bool ck0 = (key < r0.vis) & notseed, ck1 = (key < r1.vis) & notseed;
      // U >= the threshold's float floor keeps every key whose record
      // (U, key) reaches the threshold (and at most a few equal-bound keys
      // below it, which the refine drops)
      const uint64_t m0 = __ballot(ck0 & (U0 >= r0.thr_f));
      const uint64_t m1 = __ballot(ck1 & (U1 >= r1.thr_f));
      if constexpr (kBounds) {
        if (ck0 && valid0) pa.st_ub[row0 * (size_t)N + key] = U0;
        if (ck1 && valid1) pa.st_ub[row1 * (size_t)N + key] = U1;
      }
      screened0 += __popcll(__ballot(ck0));
      screened1 += __popcll(__ballot(ck1));
      survived0 += __popcll(m0);
      survived1 += __popcll(m1);
      pend0 = lane == pr ? m0 : pend0;
      pend1 = lane == pr ? m1 : pend1;
    }
    pend_w = (ts - k0) / 64;
    wait_vmem_all();  // this wave's loads of tile ti + kAhead and its bitmask stores have landed
    __syncthreads();
    cur = nxt;
  }
  flush_words();
  if (lane == 0) {
    if (valid0) {
      pa.ctl[row0].screened += screened0;
      pa.ctl[row0].survived += survived0;
    }
    if (valid1) {
      pa.ctl[row1].screened += screened1;
      pa.ctl[row1].survived += survived1;
    }
  }
}

// ---------------------------------------------------------------- 3-4. refine, select

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

// One wave per row, kRefineWaves rows per workgroup, no workgroup barrier:
// the survivors of keys [k0, k1) listed in the row's bitmask are rescored
// with all heads, 32 at a time, the next batch's key rows loading while the
// current batch is scored; records that reach the threshold become
// candidates, and every 32 kept records raise the threshold.  `final`: after
// the last chunk, select the row's exact Top-K and write the statistics;
// otherwise save the row's state for the next chunk.  kCompact: candidates
// are compact records, and the final select resolves the boundary code by
// rescoring its keys.
template <int DT, bool kCompact>
__global__ __launch_bounds__(kRefineWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_refine(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ qsc, const float* __restrict__ ksc, const int32_t* __restrict__ pos, int Q, int N,
    size_t R, int k0, int k1, int final_chunk, int topk, int cap, uint64_t* __restrict__ cand,
    int32_t* __restrict__ out_idx, float* __restrict__ out_score, PruneArgs pa) {
  constexpr int RB = Frag<DT>::kRowBytes;
  __shared__ __align__(16) uint32_t hist[kRefineWaves][256];
  __shared__ uint64_t stage[kRefineWaves][kStage];
  __shared__ int32_t queue[kRefineWaves][kQueue];
  __shared__ __align__(16) float wrow[kRefineWaves][kHeads];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * kRefineWaves + wave;
  if (row >= R) return;  // whole wave; the waves share nothing
  const int b = (int)(row / (size_t)Q);
  const bool recover = pa.flag[row] != 0;
  PruneRowCtl c = pa.ctl[row];
  if (recover) {  // the streaming Top-K recomputes the row afterwards
    if (final_chunk && lane == 0) {
      if (pa.st_tau) pa.st_tau[row] = c.tau;
      if (pa.st_screened) pa.st_screened[row] = c.reason ? c.screened : 0;
      if (pa.st_surv) pa.st_surv[row] = c.reason ? c.survived : 0;
      if (pa.st_rec) pa.st_rec[row] = (uint8_t)(c.reason ? c.reason : 1);
    }
    return;
  }
  uint32_t* my_hist = hist[wave];
  uint64_t* my_stage = stage[wave];
  int32_t* my_q = queue[wave];
  const uint32_t* gh = pa.hist + row * 256;
  for (int i = lane; i < 256; i += 64) my_hist[i] = gh[i];
  RowState rs{cand + row * (size_t)cap, c.cnt, 0, c.thr, c.base, c.shift, c.added};
  const Code32 code{c.cbase, c.cshift, key_bits(N)};
  RowState32 rc{reinterpret_cast<uint32_t*>(cand + row * (size_t)cap) + cap,
                c.cnt, 0, c.thr, code.code((uint32_t)(c.thr >> 32)), c.base, c.shift, c.added, false};
  uint32_t* my_stage32 = reinterpret_cast<uint32_t*>(my_stage);  // compact records: 2 kStage of them
  const int vis = min(max(pos[row] + 1, 0), N);
  const int end = min(k1, vis);
  const int W = end > k0 ? (end - k0 + 63) / 64 : 0;  // bitmask words to read

  Frag<DT> qa[2];
  const float* my_w = wrow[wave];
  const float qscale = (DT == kFP8) ? qsc[row] : 1.0f;
  const uint8_t* kbase = k + (size_t)b * N * RB;
  const float* kscb = (DT == kFP8) ? ksc + (size_t)b * N : nullptr;
  const int lk = lane & 31;
  if (W > 0) {  // the query block and weights
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) load_frag<DT>(qa[blk], q + (row * kHeads + 32 * blk + (lane & 31)) * RB, lane);
    wrow[wave][lane] = w[row * kHeads + lane];
  }

  if (W > 0) {
    const uint64_t* mrow = pa.mask + row * (size_t)pa.mask_stride;

    // Survivor queue my_q[qh, qn): topped up from the bitmask, kGroupWords
    // words at a time (lane j expands word g + j), whenever fewer than 64
    // keys are queued.  The next group's words are loaded one refill ahead,
    // so a refill never waits for memory behind the batches in flight.
    int qh = 0, qn = 0, g = 0;
    auto group_words = [&](int g0) { return (lane < kGroupWords && g0 + lane < W) ? mrow[g0 + lane] : 0ull; };
    uint64_t wnext = group_words(0);
    auto refill = [&]() {
      while (qn - qh < 64 && g < W) {
        if (qh > 0) {  // move the queue to the front
          const int left = qn - qh;
          for (int i = lane; i < left; i += 64) {
            const int v = my_q[qh + i];
            wave_lds_sync();
            my_q[i] = v;
          }
          wave_lds_sync();
          qn = left;
          qh = 0;
        }
        const uint64_t word = wnext;
        wnext = group_words(g + kGroupWords);
        const uint32_t n = (uint32_t)__popcll(word);
        const uint32_t incl = wave_prefix_incl(n, lane);
        int at = qn + (int)(incl - n);
        const int base_key = k0 + 64 * (g + lane);
        for (uint64_t m = word; m; m &= m - 1) my_q[at++] = base_key + (int)__builtin_ctzll(m);
        wave_lds_sync();
        qn += (int)__builtin_amdgcn_readlane((int)incl, 63);
        g += kGroupWords;
      }
    };
    // fp8 has the registers to hold the row's head weights for the whole
    // scan; bf16 would spill, so it reads them from LDS at the start of each
    // batch, ahead of its MFMAs.  Either way the weight reads stay off the
    // batch's dependent chain (measured: 1M fp8 refine 6%, 128K bf16 refine
    // 1.5% faster than reading them in the head sum).  Same FMAs, same order.
    float wl[2][16];
    if constexpr (DT == kFP8) {
      wave_lds_sync();
      load_wl(wl, my_w, lane);
    }
    // exact scores of a batch (lane l % 32: key `key`, fragment f) go to the
    // candidates if their records reach the threshold
    auto score_and_keep = [&](const Frag<DT>& f, int key, float ks, bool live) {
      float s;
      if constexpr (DT == kFP8) {
        s = combine_swap(head_partial(mma_block<DT>(qa[0], f, zero16()), mma_block<DT>(qa[1], f, zero16()), wl));
      } else {
        float wb[2][16];
        load_wl(wb, my_w, lane);
        s = combine_swap(head_partial(mma_block<DT>(qa[0], f, zero16()), mma_block<DT>(qa[1], f, zero16()), wb));
      }
      if constexpr (DT == kFP8) s = apply_scales(s, qscale, ks);
      if constexpr (kCompact) {
        if (rc.nst > 2 * kStage - 32) {
          for (int i = lane; i < rc.nst; i += 64) rc.buf[rc.cnt + i] = my_stage32[i];
          rc.cnt += rc.nst;
          rc.nst = 0;
        }
        append32(rc, make_record(s, (uint32_t)key), live, my_stage32, my_hist, code, topk, cap, lane);
        if (rc.added >= kRaiseEvery) raise32(rc, my_hist, code, topk, lane);
      } else {
        if (rs.nst > kStage - 32) {
          rs.cnt = flush_stage(rs.buf, rs.cnt, my_stage, rs.nst, lane);
          rs.nst = 0;
        }
        append_rec(rs, make_record(s, (uint32_t)key), live, my_stage, my_hist, topk, cap, lane);
        if (rs.added >= kRaiseEvery) raise_threshold(rs, my_hist, topk, lane);
      }
    };
    // Batches go through a ring of fragments: the next batches' key rows
    // are loading while one is scored (fp8: two in flight, bf16: one).  A batch is issued
    // unconditionally (an empty one reloads key 0, a valid row, never
    // scored), so the loads form one straight sequence.
    struct Batch {
      Frag<DT> f;
      int key, n;
      float ks;
    };
    auto issue = [&](Batch& bt) {
      refill();
      bt.n = min(32, qn - qh);
      bt.key = bt.n > 0 ? my_q[qh + (lk < bt.n ? lk : 0)] : 0;
      load_frag<DT>(bt.f, kbase + (size_t)bt.key * RB, lane);
      bt.ks = (DT == kFP8) ? kscb[bt.key] : 1.0f;
      qh += bt.n;
    };
    if constexpr (DT == kBF16) {  // two batches (one in flight): a third would not fit the registers
      Batch b0, b1;
      issue(b0);
      while (true) {
        if (b0.n == 0) break;
        issue(b1);
        score_and_keep(b0.f, b0.key, b0.ks, lane < b0.n);
        if (b1.n == 0) break;
        issue(b0);
        score_and_keep(b1.f, b1.key, b1.ks, lane < b1.n);
      }
    } else {
      Batch b0, b1, b2;
      issue(b0);
      issue(b1);
      while (true) {
        if (b0.n == 0) break;
        issue(b2);
        score_and_keep(b0.f, b0.key, b0.ks, lane < b0.n);
        if (b1.n == 0) break;
        issue(b0);
        score_and_keep(b1.f, b1.key, b1.ks, lane < b1.n);
        if (b2.n == 0) break;
        issue(b1);
        score_and_keep(b2.f, b2.key, b2.ks, lane < b2.n);
      }
    }
  }

  if (!final_chunk || kCompact) {  // compact records: the select runs in k_emit_compact
    uint32_t* ghw = pa.hist + row * 256;
    if constexpr (kCompact) {
      for (int i = lane; i < rc.nst; i += 64) rc.buf[rc.cnt + i] = my_stage32[i];
      rc.cnt += rc.nst;
      rc.nst = 0;
      row_mem_sync();
      for (int i = lane; i < 256; i += 64) ghw[i] = my_hist[i];
      if (lane == 0) {
        PruneRowCtl& cw = pa.ctl[row];
        cw.thr = rc.thr;
        cw.cnt = rc.cnt;
        cw.base = rc.hbase;
        cw.shift = rc.hshift;
        cw.added = rc.added;
        if (rc.dead) {  // later launches skip the row; the streaming Top-K recomputes it
          cw.reason = 3;
          pa.flag[row] = 1;
        }
      }
    } else {
      rs.cnt = flush_stage(rs.buf, rs.cnt, my_stage, rs.nst, lane);
      rs.nst = 0;
      row_mem_sync();
      for (int i = lane; i < 256; i += 64) ghw[i] = my_hist[i];
      if (lane == 0) {
        PruneRowCtl& cw = pa.ctl[row];
        cw.thr = rs.thr;
        cw.cnt = rs.cnt;
        cw.base = rs.base;
        cw.shift = rs.shift;
        cw.added = rs.added;
      }
    }
    return;
  }
  auto recover_row = [&](int reason) {  // the streaming Top-K recomputes the row
    if (lane == 0) {
      pa.flag[row] = 1;
      if (pa.st_tau) pa.st_tau[row] = c.tau;
      if (pa.st_screened) pa.st_screened[row] = c.screened;
      if (pa.st_surv) pa.st_surv[row] = c.survived;
      if (pa.st_rec) pa.st_rec[row] = (uint8_t)reason;
    }
  };
  auto row_stats = [&]() {
    if (lane == 0) {
      if (pa.st_tau) pa.st_tau[row] = c.tau;
      if (pa.st_screened) pa.st_screened[row] = c.screened;
      if (pa.st_surv) pa.st_surv[row] = c.survived;
      if (pa.st_rec) pa.st_rec[row] = 0;
    }
  };
  int32_t* oi = out_idx + row * (size_t)topk;
  float* os = out_score ? out_score + row * (size_t)topk : nullptr;
  // Every kept record reaches the row's start and every key whose record
  // does was kept, so with fewer than K of them (possible only after a
  // raised start) the K-th best record lies below the start: the streaming
  // Top-K recomputes the row.
  if (rs.cnt + rs.nst < topk && c.raised) {
    recover_row(2);
    return;
  }
  emit_topk_d8(rs.buf, rs.cnt, my_stage, rs.nst, my_hist, topk, oi, os, lane);
  row_stats();
}

// Final select of the rows with compact records, after the last chunk's
// refine (one wave per row): radix select over the codes finds the Top-K's
// boundary code; the records above it are in.  If only part of the boundary
// code's records are needed, or the scores are requested, the keys in
// question are rescored with all heads by the shared routine into exact
// 64-bit records (in the first half of the row's buffer) and those are
// selected exactly (DoSA reading notes, annotation TMIF4XYF: records above
// the boundary code are kept, the boundary is resolved by the original
// scores).  Rows that cannot be resolved in the buffer, and missed raised
// starts, are flagged for the streaming Top-K.
template <int DT>
__global__ __launch_bounds__(kRefineWaves * 64) void k_emit_compact(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ qsc, const float* __restrict__ ksc, int Q, int N, size_t R, int topk, int cap,
    uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_score, PruneArgs pa) {
  constexpr int RB = Frag<DT>::kRowBytes;
  __shared__ __align__(16) uint32_t hist[kRefineWaves][256];
  __shared__ int32_t queue[kRefineWaves][kQueue];
  __shared__ __align__(16) float wrow[kRefineWaves][kHeads];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * kRefineWaves + wave;
  if (row >= R) return;  // whole wave; the waves share nothing
  const int b = (int)(row / (size_t)Q);
  const PruneRowCtl c = pa.ctl[row];
  auto stats = [&](int reason, bool counts) {
    if (lane == 0) {
      if (pa.st_tau) pa.st_tau[row] = c.tau;
      if (pa.st_screened) pa.st_screened[row] = counts ? c.screened : 0;
      if (pa.st_surv) pa.st_surv[row] = counts ? c.survived : 0;
      if (pa.st_rec) pa.st_rec[row] = (uint8_t)reason;
    }
  };
  if (pa.flag[row]) {  // flagged before (plan, seeds, forced, or a buffer the refine could not cut)
    stats(c.reason ? c.reason : 1, c.reason != 0);
    return;
  }
  auto recover_row = [&](int reason) {
    if (lane == 0) pa.flag[row] = 1;
    stats(reason, true);
  };
  const Code32 code{c.cbase, c.cshift, key_bits(N)};
  const uint32_t* buf = reinterpret_cast<const uint32_t*>(cand + row * (size_t)cap) + cap;
  const int cnt = c.cnt;
  if (cnt < topk && c.raised) {  // fewer than K records reach the raised start: it was missed
    recover_row(2);
    return;
  }
  uint32_t* my_hist = hist[wave];
  int32_t* my_q = queue[wave];
  int32_t* oi = out_idx + row * (size_t)topk;
  float* os = out_score ? out_score + row * (size_t)topk : nullptr;
  const int need = min(topk, cnt);
  const bool all = os != nullptr;
  CodeCut sel{0u, 0u, 0u};
  int nres = 0;
  if (need > 0) {
    sel = select_code32(buf, cnt, (uint32_t)need, code.kb, my_hist, 0u, lane);
    nres = all ? (int)(sel.above + sel.at) : (sel.above + sel.at == (uint32_t)need ? 0 : (int)sel.at);
    if (nres > cap / 2) {
      recover_row(3);
      return;
    }
  }
  int base = 0;
  auto emit_codes = [&](bool above_only) {  // the records of code >= cmin (> cmin)
    for (int i0 = 0; i0 < cnt; i0 += 64) {
      const int i = i0 + lane;
      const uint32_t r = i < cnt ? buf[i] : 0u;
      const uint32_t rc = r >> code.kb;
      const bool keep = i < cnt && (above_only ? rc > sel.cmin : rc >= sel.cmin);
      const uint64_t bal = __ballot(keep);
      if (keep)
        oi[base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] =
            (int32_t)code.key(r);
      base += __popcll(bal);
    }
  };
  if (nres == 0) {
    emit_codes(false);  // exactly need of them
  } else {
    Frag<DT> qa[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) load_frag<DT>(qa[blk], q + (row * kHeads + 32 * blk + (lane & 31)) * RB, lane);
    wrow[wave][lane] = w[row * kHeads + lane];
    const float* my_w = wrow[wave];
    const float qscale = (DT == kFP8) ? qsc[row] : 1.0f;
    const uint8_t* kbase = k + (size_t)b * N * RB;
    const float* kscb = (DT == kFP8) ? ksc + (size_t)b * N : nullptr;
    const int lk = lane & 31;
    uint64_t* scratch = cand + row * (size_t)cap;
    int nscr = 0, qn = 0;
    auto score_queue = [&]() {  // exact records of the queued keys, 32 at a time
      for (int i0 = 0; i0 < qn; i0 += 32) {
        const int n = min(32, qn - i0);
        const int key = my_q[i0 + (lk < n ? lk : 0)];
        Frag<DT> f;
        load_frag<DT>(f, kbase + (size_t)key * RB, lane);
        const float ks = (DT == kFP8) ? kscb[key] : 1.0f;
        float sc = combine_swap(query_partial_w<DT>(qa, f, my_w, lane));
        if constexpr (DT == kFP8) sc = apply_scales(sc, qscale, ks);
        if (lane < n) scratch[nscr + lane] = make_record(sc, (uint32_t)key);
        nscr += n;
      }
      qn = 0;
      wave_lds_sync();
    };
    for (int i0 = 0; i0 < cnt; i0 += 64) {
      const int i = i0 + lane;
      const uint32_t r = i < cnt ? buf[i] : 0u;
      const uint32_t rc = r >> code.kb;
      const bool take = i < cnt && (all ? rc >= sel.cmin : rc == sel.cmin);
      const uint64_t bal = __ballot(take);
      if (take)
        my_q[qn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] =
            (int32_t)code.key(r);
      qn += __popcll(bal);
      wave_lds_sync();
      if (qn > kQueue - 64) score_queue();
    }
    if (qn > 0) score_queue();
    row_mem_sync();
    const SelectResult s2 =
        select_records_d8(scratch, nscr, (uint32_t)(all ? need : need - (int)sel.above), my_hist, true, 0, lane);
    if (!all) emit_codes(true);  // the records above the boundary code
    for (int i0 = 0; i0 < nscr; i0 += 64) {
      const int i = i0 + lane;
      const uint64_t r = i < nscr ? scratch[i] : 0ull;
      const bool keep = i < nscr && (r & s2.mask) >= s2.prefix;
      const uint64_t bal = __ballot(keep);
      const int at = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (keep) {
        oi[at] = (int32_t)record_key(r);
        if (os) os[at] = record_score(r);
      }
      base += __popcll(bal);
    }
  }
  for (int j = need + lane; j < topk; j += 64) {
    oi[j] = -1;
    if (os) os[j] = -INFINITY;
  }
  stats(0, true);
}

#define DSA_SCREEN_KERNEL(DT_, B_)                                                                                \
  template __global__ void k_screen<DT_, B_>(const float* __restrict__, const uint8_t* __restrict__,             \
                                             const float* __restrict__, const int32_t* __restrict__, int, int, int, \
                                             int, PruneArgs);
DSA_SCREEN_KERNEL(kBF16, false)
DSA_SCREEN_KERNEL(kBF16, true)
DSA_SCREEN_KERNEL(kFP8, false)
DSA_SCREEN_KERNEL(kFP8, true)
#undef DSA_SCREEN_KERNEL

__global__ void k_fill_nan(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = __builtin_nanf("");
}

// Key chunks of the screen/refine schedule: the first two of
// max(4096, N / 32) keys (rounded up to 4096), then lengths doubling, none
// longer than kPruneChunkBytes of key rows.  Boundaries are multiples of
// 4096: whole screen tiles and bitmask words.
std::vector<std::pair<int, int>> prune_chunks(int N, int row_bytes) {
  const int max_len = kPruneChunkBytes / row_bytes;
  std::vector<std::pair<int, int>> out;
  int len = std::min(max_len, std::max(4096, (N / 32 + 4095) / 4096 * 4096));
  for (int s = 0; s < N;) {
    const int e = (int)std::min<int64_t>((int64_t)s + len, N);
    out.emplace_back(s, e);
    s = e;
    if (out.size() >= 2) len = std::min(2 * len, max_len);
  }
  return out;
}

int prune_mask_words(int N, int row_bytes) {
  int mx = 0;
  for (const auto& c : prune_chunks(N, row_bytes)) mx = std::max(mx, c.second - c.first);
  // the screen writes whole tiles (up to 128 keys, two words) past a
  // chunk's last key
  return (mx + 127) / 128 * 2;
}

hipError_t launch_topk_pruned(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx, float* out_score,
                              const PrunedBuffers& pb, hipStream_t st) {
  const size_t R = (size_t)p.B * p.Q;
  PruneArgs pa{pb.plan_rows,   pb.plan_coef,    pb.plan_misc,    pb.plan_flag,   pb.knorm,
               pb.seeds,       pb.seed_stride,  pb.seed_bits,    pb.bits_stride, pb.seed_pos,
               pb.raised_start, pb.compact,     pb.seed_top_idx, pb.seed_top_score, pb.ctl, pb.hist,
               pb.mask,        pb.mask_stride,  pb.st_tau,       pb.st_screened, pb.st_surv,
               pb.st_rec,      pb.st_ub};
  if (pb.st_ub) {
    const size_t n = R * p.N;
    hipLaunchKernelGGL(k_fill_nan, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pb.st_ub, n);
  }
  const dim3 rgrid((unsigned)((R + kRefineWaves - 1) / kRefineWaves));
  int slot = prof_open("k_prune_init", st);
  hipLaunchKernelGGL(k_prune_init, rgrid, dim3(kRefineWaves * 64), 0, st, p.pos, p.Q, p.N, R, topk, cap, cand, pa);
  prof_close(slot, st);

  using ScreenKern = void (*)(const float*, const uint8_t*, const float*, const int32_t*, int, int, int, int,
                              PruneArgs);
  const ScreenKern screen = p.dtype == kBF16 ? (pb.st_ub ? k_screen<kBF16, true> : k_screen<kBF16, false>)
                                             : (pb.st_ub ? k_screen<kFP8, true> : k_screen<kFP8, false>);
  using RefineKern = void (*)(const uint8_t*, const uint8_t*, const float*, const float*, const float*,
                              const int32_t*, int, int, size_t, int, int, int, int, int, uint64_t*, int32_t*, float*,
                              PruneArgs);
  const RefineKern refine = p.dtype == kBF16 ? (pb.compact ? k_refine<kBF16, true> : k_refine<kBF16, false>)
                                             : (pb.compact ? k_refine<kFP8, true> : k_refine<kFP8, false>);
  const dim3 sgrid((unsigned)((p.Q + 2 * kScreenWaves - 1) / (2 * kScreenWaves)), p.B);
  const auto chunks = prune_chunks(p.N, p.dtype == kBF16 ? 256 : 128);
  for (size_t c = 0; c < chunks.size(); ++c) {
    const int k0 = chunks[c].first, k1 = chunks[c].second;
    const int fin = c + 1 == chunks.size() ? 1 : 0;
    slot = prof_open("k_screen", st);
    hipLaunchKernelGGL(screen, sgrid, dim3(kScreenWaves * 64), 0, st, p.q_scale, p.k, p.k_scale, p.pos, p.Q, p.N, k0,
                       k1, pa);
    prof_close(slot, st);
    slot = prof_open("k_refine", st);
    hipLaunchKernelGGL(refine, rgrid, dim3(kRefineWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, R, k0, k1, pb.compact ? 0 : fin, topk, cap, cand, out_idx, out_score, pa);
    prof_close(slot, st);
  }
  if (pb.compact) {
    slot = prof_open("k_emit_compact", st);
    if (p.dtype == kBF16)
      hipLaunchKernelGGL(k_emit_compact<kBF16>, rgrid, dim3(kRefineWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale,
                         p.k_scale, p.Q, p.N, R, topk, cap, cand, out_idx, out_score, pa);
    else
      hipLaunchKernelGGL(k_emit_compact<kFP8>, rgrid, dim3(kRefineWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale,
                         p.k_scale, p.Q, p.N, R, topk, cap, cand, out_idx, out_score, pa);
    prof_close(slot, st);
  }
  // recovery: flagged rows by the unpruned streaming Top-K
  return launch_topk_stream_rows(p, topk, cap, cand, out_idx, out_score, pb.plan_flag, "k_topk_stream_recover", st);
}

}  // namespace dsa
