// stream_common.h -- pieces shared by the streaming Top-K kernels (unpruned
// and pruned): LDS key tiles, per-row candidate bookkeeping, final emit.
#pragma once
#include <math.h>

#include "score_tile.h"
#include "select.h"

namespace dsa {

constexpr int kWaves = 8;           // query rows per workgroup, one per wave
constexpr int kTileBytes = 16384;   // one LDS key tile (64 bf16 or 128 fp8 keys)

// LDS key tile layout: chunk-major with one chunk of padding per chunk row.
// 16-byte chunk c of tile key r lives at chunk index c * (KT + 1) + r, so
//  - the 32 (or 16) lanes that read chunk c of consecutive keys read one
//    contiguous run (conflict-free), and a lane's successive chunks are a
//    constant stride apart (immediate ds_read offsets from one base address);
//  - the 16 (bf16) / 8 (fp8) threads that store the chunks of one key hit
//    different banks, the row pitch being (KT + 1) * 16 bytes.
constexpr int kTileChunks = 1040;  // max over dtypes of (chunks per key) * (KT + 1)

template <int DT>
__device__ __forceinline__ int tile_chunk(int key, int c) {
  constexpr int KT = kTileBytes / Frag<DT>::kRowBytes;
  return c * (KT + 1) + key;
}

// Fragment of key `key` (tile-relative) from an LDS tile.
template <int DT>
__device__ __forceinline__ void load_frag_lds(Frag<DT>& f, const u32x4* tile, int key, int lane) {
  constexpr int CPL = Frag<DT>::kLaneBytes / 16;  // chunks per lane
  const int c0 = (lane >> 5) * CPL;
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = tile[tile_chunk<DT>(key, c0 + i)];
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 lo = tile[tile_chunk<DT>(key, c0 + 2 * i)], hi = tile[tile_chunk<DT>(key, c0 + 2 * i + 1)];
      f.v[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
}

// Candidate bookkeeping of one row (one wave): records are appended to a
// small LDS stage during a tile and flushed to the row's global buffer at the
// start of the next tile, so the tile-end wait for the next key tile never
// waits on fresh candidate stores.  H1 (the top-digit histogram) counts
// every record in the buffer and the stage.  State: cnt records in buf, nst
// in the stage, running threshold thr (records below it cannot be in the
// Top-K).
__device__ __forceinline__ int flush_stage(uint64_t* buf, int cnt, const uint64_t* stage, int nst, int lane) {
  for (int i = lane; i < nst; i += 64) buf[cnt + i] = stage[i];
  return cnt + nst;
}

struct Cut {
  int cnt;
  uint64_t thr;
};

// Cut the row's candidates (buffer + stage) back to at most `goal` (>= topk)
// records and raise the threshold to the cut's boundary; goal == topk keeps
// exactly the best topk, so the threshold becomes the K-th best record seen.
static __device__ __noinline__ Cut cut_candidates(uint64_t* buf, int cnt, const uint64_t* stage, int nst, uint32_t* hist,
                                           int topk, int goal, int lane) {
  cnt = flush_stage(buf, cnt, stage, nst, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  const SelectResult sel = select_records(buf, cnt, (uint32_t)topk, hist, false, (uint32_t)goal, lane);
  return {compact_records(buf, cnt, sel, hist, lane), sel.prefix};
}

// Write the row's exact Top-K (min(topk, cnt) indices, then -1 padding).
static __device__ __noinline__ void emit_topk(uint64_t* buf, int cnt, const uint64_t* stage, int nst, uint32_t* hist,
                                       int topk, int32_t* oi, float* os, int lane) {
  cnt = flush_stage(buf, cnt, stage, nst, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  const int need = min(topk, cnt);
  SelectResult sel = {0, 0, 0};
  if (need > 0) sel = select_records(buf, cnt, (uint32_t)need, hist, true, 0, lane);
  int base = 0;
  for (int i0 = 0; i0 < cnt; i0 += 64) {
    const int i = i0 + lane;
    uint64_t r = 0;
    bool keep = false;
    if (i < cnt) {
      r = buf[i];
      keep = (r & sel.mask) >= sel.prefix;
    }
    const uint64_t bal = __ballot(keep);
    const uint32_t before =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (keep) {
      oi[base + before] = (int32_t)record_key(r);
      if (os) os[base + before] = record_score(r);
    }
    base += __popcll(bal);
  }
  for (int j = need + lane; j < topk; j += 64) {
    oi[j] = -1;
    if (os) os[j] = -INFINITY;
  }
}

// The same pair for rows without the incremental histogram (8-bit digits).
static __device__ __noinline__ Cut cut_candidates_d8(uint64_t* buf, int cnt, const uint64_t* stage, int nst,
                                                     uint32_t* hist, int topk, int goal, int lane) {
  cnt = flush_stage(buf, cnt, stage, nst, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  const SelectResult sel = select_records_d8(buf, cnt, (uint32_t)topk, hist, false, (uint32_t)goal, lane);
  return {compact_records_d8(buf, cnt, sel, lane), sel.prefix};
}

static __device__ __noinline__ void emit_topk_d8(uint64_t* buf, int cnt, const uint64_t* stage, int nst,
                                                 uint32_t* hist, int topk, int32_t* oi, float* os, int lane) {
  cnt = flush_stage(buf, cnt, stage, nst, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  const int need = min(topk, cnt);
  SelectResult sel = {0, 0, 0};
  if (need > 0) sel = select_records_d8(buf, cnt, (uint32_t)need, hist, true, 0, lane);
  int base = 0;
  for (int i0 = 0; i0 < cnt; i0 += 64) {
    const int i = i0 + lane;
    uint64_t r = 0;
    bool keep = false;
    if (i < cnt) {
      r = buf[i];
      keep = (r & sel.mask) >= sel.prefix;
    }
    const uint64_t bal = __ballot(keep);
    const uint32_t before =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (keep) {
      oi[base + before] = (int32_t)record_key(r);
      if (os) os[base + before] = record_score(r);
    }
    base += __popcll(bal);
  }
  for (int j = need + lane; j < topk; j += 64) {
    oi[j] = -1;
    if (os) os[j] = -INFINITY;
  }
}

// Next key tile: each thread fetches two 16-byte chunks into registers at the
// start of a tile and stores them (swizzled) into the other LDS buffer at its
// end, so the fetch latency hides behind the current tile's MFMAs.  Keys at
// or past N read key N-1 (never scored: visibility masks them).
template <int DT>
struct TileFetch {
  static constexpr int CPR = Frag<DT>::kRowBytes / 16;
  static constexpr int CHUNKS = kTileBytes / 16;
  static constexpr int PER_THREAD = CHUNKS / (kWaves * 64);
  static constexpr int KT = kTileBytes / Frag<DT>::kRowBytes;
  u32x4 v[PER_THREAD];
  float ks;   // fp8 key scale of tile row tid (tid < KT)
  float kn;   // key norm of tile row tid (pruned path, tid < KT)
  uint32_t sbw;  // seed-bitmap word tid (pruned path, tid < KT / 32)

  // Tile rows ts..ts+KT-1 of the key sequence; with `gidx`, tile row r is key
  // gidx[min(ts + r, nidx - 1)] (a gathered tile), else key min(ts + r, N - 1).
  // `knorm` / `sbits` (pruned path) also stage each row's |k| and the seed
  // bitmap words of a contiguous tile.
  __device__ __forceinline__ void fetch(const uint8_t* kbase, const float* kscb, int ts, int N, int tid,
                                        const int32_t* gidx = nullptr, int nidx = 0, const float* knorm = nullptr,
                                        const uint32_t* sbits = nullptr) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * kWaves * 64;
      const int key = c / CPR, ch = c % CPR;
      const int gk = gidx ? gidx[min(ts + key, nidx - 1)] : min(ts + key, N - 1);
      v[j] = *reinterpret_cast<const u32x4*>(kbase + (size_t)gk * Frag<DT>::kRowBytes + ch * 16);
    }
    if (tid < KT) {
      const int gk = gidx ? gidx[min(ts + tid, nidx - 1)] : min(ts + tid, N - 1);
      if constexpr (DT == kFP8) ks = kscb[gk];
      if (knorm) kn = knorm[gk];
    }
    if (sbits && tid < KT / 32) sbw = sbits[min(ts / 32 + tid, (N - 1) / 32)];
  }
  __device__ __forceinline__ void commit(u32x4* tile, float* kst, int tid, float* knt = nullptr,
                                         uint32_t* sbt = nullptr) const {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * kWaves * 64;
      tile[tile_chunk<DT>(c / CPR, c % CPR)] = v[j];
    }
    if (tid < KT) {
      if constexpr (DT == kFP8) kst[tid] = ks;
      if (knt) knt[tid] = kn;
    }
    if (sbt && tid < KT / 32) sbt[tid] = sbw;
  }
};

}  // namespace dsa
