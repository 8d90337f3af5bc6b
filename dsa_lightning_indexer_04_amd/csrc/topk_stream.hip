// topk_stream.hip -- fused scoring + exact streaming Top-K for prefill blocks.
//
// The indexer must score the whole causal prefix of every query before it
// knows its Top-K (DeepSeek DSA FLOPs notes, remark at the end of
// "Full-prefix index scoring"); this kernel does that without ever storing
// the score matrix.  Each row keeps a running threshold and a candidate
// buffer of records in global memory; a key is appended only if its record
// is not below the threshold.  Every 256 kept records the threshold rises to
// within one bin of the K-th best record seen, read off a per-row histogram
// of the kept score codes; when the buffer fills it is compacted to the
// records above the threshold and, if still too full, cut by radix select.
// At the end the buffer's best min(topk, visible) records are the exact
// Top-K.
//
// Organisation (gfx950):
//   workgroup = 4 waves = 4 consecutive query rows of one sequence, one row
//               per wave held in registers as MFMA A fragments (64 heads x
//               128 dims) plus its head weights; two workgroups per CU, two
//               waves per SIMD, so one wave's MFMAs overlap the other's fp32
//               epilogue and one workgroup's tile barrier the other's work;
//   key tiles (16 KiB: 64 bf16 or 128 fp8 keys) rotate through three LDS
//   slots: the tile after next streams from global memory straight into
//   LDS while the current one is scored, in a padded key-major layout so
//   the column reads are bank-conflict free; the workgroup's 4 waves read
//   each tile, and each wave's key fragment for the next 32 keys is read
//   while the current 32 are multiplied.
//   After the head sum and one cross-half exchange every lane holds the
//   score of key l%32; two blocks are appended together, one key per lane.
//   Workgroups are issued longest-prefix first (causal imbalance).
#include <math.h>

#include "kernels.h"
#include "stream_common.h"

namespace dsa {

constexpr int kWaves = 4;           // query rows per workgroup, one per wave (two workgroups per CU)
constexpr int kTileBytes = 16384;   // key bytes of one LDS tile: 64 bf16 or 128 fp8 keys
constexpr int kSlots = 3;           // LDS key-tile slots
// Kept records between threshold raises.  A raise is a wave-wide prefix sum
// over the histogram; early in a row, when most keys are kept, raising every
// 256 records instead of every 32 lets the threshold lag a little but costs
// far fewer raises (the prefill blocks ran 1-3% faster).
constexpr int kStreamRaiseEvery = 256;

template <int DT>
struct BlockAcc {
  f32x16 s0, s1;  // heads 0..31 / 32..63 of one query against 32 keys
};

// Append the records of two scored 32-key blocks at once: lane l holds the
// score of key `key` (the earlier block in lanes 0..31, the later one in
// 32..63; `live` masks keys that are not visible).  A key is kept if its
// score reaches thr_f, the float floor of the threshold record: that keeps
// every record >= thr (and at most a few equal-score records below it,
// which the exact selections drop).  The stores are branch-free, so the
// scheduler can overlap them with the next block's MFMAs: every lane stores
// its record, the kept ones to the next stage slots and the others to their
// own slot of the stage's scratch tail (stage[dummy + lane]).  The stage has
// room: the caller flushes it at tile boundaries.
__device__ __forceinline__ void append_pair(RowState& rs, float thr_f, float s, int key, bool live, uint64_t* stage,
                                            int dummy, int lane) {
  const bool take = live && s >= thr_f;
  const uint64_t bal = __ballot(take);
  const int before =
      (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
  const uint64_t rec = make_record(s, (uint32_t)key);
  stage[take ? rs.nst + before : dummy + lane] = rec;
  const int n = __popcll(bal);
  rs.nst += n;
  rs.added += n;
}

// Tile-boundary bookkeeping of a row: count the staged records in the
// threshold histogram (here, where no key-tile load is in flight, rather than
// at each append) and flush them to the buffer; every
// kStreamRaiseEvery kept records raise the threshold from the histogram (to within
// one bin of the K-th best record seen, no buffer traffic); if `room` more
// records could overflow the buffer, rebuild: keep the records >= thr, cut
// them by radix select when too many remain, and rebuild the histogram with
// bins fitted to the kept records.
__device__ __forceinline__ void tile_bookkeeping(RowState& rs, float& thr_f, uint64_t* stage, uint32_t* hist,
                                                 int topk, int cap, int room, int lane) {
  if (rs.nst) {
    for (int i = lane; i < rs.nst; i += 64) atomicAdd(&hist[thr_bin((uint32_t)(stage[i] >> 32), rs.base, rs.shift)], 1u);
    rs.cnt = flush_stage(rs.buf, rs.cnt, stage, rs.nst, lane);
    rs.nst = 0;
  }
  if (rs.added >= kStreamRaiseEvery) {
    raise_threshold(rs, hist, topk, lane);
    thr_f = record_floor(rs.thr);
  }
  if (rs.cnt > cap - room) {
    apply_rebuild(rs, rebuild_candidates(rs.buf, rs.cnt, stage, 0, hist, rs.thr, topk, cut_goal(topk, cap), lane));
    thr_f = record_floor(rs.thr);
    rs.added = kStreamRaiseEvery;  // raise from the refitted bins at the next tile
  }
}

template <int DT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_topk_stream(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ qsc, const float* __restrict__ ksc, const int32_t* __restrict__ pos, int Q, int N,
    int topk, int cap, uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_score,
    const int32_t* __restrict__ row_flag) {
  using Tile = DirectTile<DT, kTileBytes, kWaves>;
  constexpr int RB = Frag<DT>::kRowBytes;
  constexpr int KT = Tile::KT;   // keys per tile
  constexpr int NSB = KT / 32;   // 32-key blocks per tile (even)
  __shared__ u32x4 ktile[kSlots][direct_slots(kTileBytes)];
  __shared__ float kscale_tile[kSlots][KT];
  __shared__ __align__(16) uint32_t hist[kWaves][256];  // radix-select bins (8-bit digits), threshold histogram
  __shared__ uint64_t stage[kWaves][KT + 64];  // KT records + 64 scratch slots
  __shared__ uint32_t toff[kWaves][Tile::PER_WAVE * 64];  // tile-load source offsets

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = gridDim.x - 1 - blockIdx.x;  // longest prefixes first
  const int b = blockIdx.y;
  const int t = group * kWaves + wave;
  // with row_flag, only the flagged rows are computed (and a workgroup with
  // none returns at once)
  auto taken = [&](int tj) { return tj < Q && (!row_flag || row_flag[(size_t)b * Q + tj] != 0); };
  const bool valid = taken(t);
  const size_t row = (size_t)b * Q + min(t, Q - 1);
  const int vis = valid ? min(max(pos[row] + 1, 0), N) : 0;
  int wg_vis = 0;
  bool any = false;
  for (int j = 0; j < kWaves; ++j) {
    const int tj = group * kWaves + j;
    if (taken(tj)) {
      any = true;
      wg_vis = max(wg_vis, min(max(pos[(size_t)b * Q + tj] + 1, 0), N));
    }
  }
  if (!any) return;  // workgroup-uniform, before any barrier

  QuerySide<DT> qs;
  load_query<DT>(qs, q + row * kHeads * RB, w + row * kHeads, lane);
  const float qscale = (DT == kFP8) ? qsc[row] : 1.0f;

  uint32_t* my_hist = hist[wave];
  uint64_t* my_stage = stage[wave];
  // threshold histogram: coarse bins over the whole code range (code >> 24)
  // until the first rebuild
  for (int i = lane; i < 256; i += 64) my_hist[i] = 0u;
  RowState rs{cand + row * (size_t)cap, 0, 0, 0, 0u, 24, 0};
  float thr_f = -INFINITY;
  const uint8_t* kbase = k + (size_t)b * N * RB;
  const float* kscb = (DT == kFP8) ? ksc + (size_t)b * N : nullptr;

  // Key tiles rotate through kSlots LDS slots: while tile ti is scored, tile
  // ti+1 already sits in the next slot (so the last block of tile ti can
  // prefetch the first fragment of tile ti+1) and tile ti+2 streams from
  // global memory straight into the slot tile ti-1 used.
  Tile tl;
  tl.init(toff[wave], wave, lane);
  const int ntiles = (wg_vis + KT - 1) / KT;
  for (int ti = 0; ti < min(ntiles, 2); ++ti) {
    tl.load(ktile[ti], kbase, ti * KT, N, lane);
    if constexpr (DT == kFP8) tl.load_words(kscale_tile[ti], kscb, ti * KT, N, lane);
  }
  wait_vmem_all();
  __syncthreads();

  // Software pipeline over 32-key blocks j = 0, 1, ...: step j issues block
  // j's MFMAs (key fragment f, loaded during step j-1) interleaved with the
  // head sum of block j-1 (from registers) and the reload of f with block
  // j+1.  Blocks are appended in pairs: an odd step keeps block j-1's score,
  // an even step appends blocks j-2 and j-1 (64 consecutive keys, one per
  // lane).  Every step runs the same straight-line code; keys past the row's
  // visible prefix and the blocks before 0 are masked at the append.
  // acc[j & 1] holds block j, kscl[j & 1] its fp8 key scales.
  BlockAcc<DT> acc[2];
  acc[0].s0 = acc[0].s1 = acc[1].s0 = acc[1].s1 = zero16();
  float kscl[2] = {1.0f, 1.0f};
  float s_prev = 0.0f;
  const int lk = lane & 31;
  Frag<DT> f;
  Tile::frag(f, ktile[0], lk, lane);
  int cur = 0;  // slot of tile ti
  for (int ti = 0; ti < ntiles; ++ti) {
    const int nxt = cur == kSlots - 1 ? 0 : cur + 1;       // slot of tile ti+1
    const int spare = nxt == kSlots - 1 ? 0 : nxt + 1;     // slot of tile ti-1, refilled with ti+2
    tile_bookkeeping(rs, thr_f, my_stage, my_hist, topk, cap, KT, lane);
    if (ti + 2 < ntiles) {
      tl.load(ktile[spare], kbase, (ti + 2) * KT, N, lane);
      if constexpr (DT == kFP8) tl.load_words(kscale_tile[spare], kscb, (ti + 2) * KT, N, lane);
    }
#pragma unroll
    for (int sub = 0; sub < NSB; ++sub) {
      const int j = ti * NSB + sub;
      BlockAcc<DT>& an = acc[sub & 1];
      const BlockAcc<DT>& ap = acc[(sub & 1) ^ 1];
      // the next block: the same tile's next 32 keys, else the next tile's
      // first (the last tile's last block reloads keys it never scores)
      const u32x4* ntile = sub + 1 < NSB ? ktile[cur] : ktile[ti + 1 < ntiles ? nxt : cur];
      const int nkey = sub + 1 < NSB ? 32 * (sub + 1) + lk : lk;
      float s = combine_single(pipelined_partial<DT>(qs, f, ap.s0, ap.s1, an.s0, an.s1,
                                                     [&](int i) { Tile::frag_step(f, ntile, nkey, i, lane); }));
      if constexpr (DT == kFP8) {
        s = apply_scales(s, qscale, kscl[(sub & 1) ^ 1]);
        kscl[sub & 1] = kscale_tile[cur][32 * sub + lk];
      }
      if (sub & 1) {
        s_prev = s;
      } else {
        const int key = 32 * (j - 2) + lane;
        append_pair(rs, thr_f, lane < 32 ? s_prev : s, key, j >= 2 && key < vis, my_stage, KT, lane);
      }
    }
    wait_vmem_all();  // this wave's loads of tile ti+2 have landed
    __syncthreads();
    cur = nxt;
  }
  if (!valid) return;
  if (ntiles > 0) {  // drain: the last block, j = ntiles * NSB - 1 (odd), is in acc[1]
    tile_bookkeeping(rs, thr_f, my_stage, my_hist, topk, cap, 64, lane);
    float s = combine_single(head_partial(acc[1].s0, acc[1].s1, qs.wl));
    if constexpr (DT == kFP8) s = apply_scales(s, qscale, kscl[1]);
    const int key = 32 * (ntiles * NSB - 2) + lane;
    append_pair(rs, thr_f, lane < 32 ? s_prev : s, key, key < vis, my_stage, KT, lane);
  }
  emit_topk_d8(rs.buf, rs.cnt, my_stage, rs.nst, my_hist, topk, out_idx + row * (size_t)topk,
               out_score ? out_score + row * (size_t)topk : nullptr, lane);
}

hipError_t launch_topk_stream_rows(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx,
                                   float* out_score, const int32_t* row_flag, const char* prof_name, hipStream_t st) {
  const int prof_slot = prof_open(prof_name, st);
  dim3 grid((p.Q + kWaves - 1) / kWaves, p.B);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_topk_stream<kBF16>, grid, dim3(kWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, topk, cap, cand, out_idx, out_score, row_flag);
  else
    hipLaunchKernelGGL(k_topk_stream<kFP8>, grid, dim3(kWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, topk, cap, cand, out_idx, out_score, row_flag);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

hipError_t launch_topk_stream(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx,
                              float* out_score, hipStream_t st) {
  return launch_topk_stream_rows(p, topk, cap, cand, out_idx, out_score, nullptr, "k_topk_stream", st);
}

}  // namespace dsa
