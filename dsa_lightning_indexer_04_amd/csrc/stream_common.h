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

// k-step i of a key fragment from an LDS tile (the slice load_frag_lds puts
// in f.v[i]).
template <int DT>
__device__ __forceinline__ void load_frag_step_lds(Frag<DT>& f, const u32x4* tile, int key, int i, int lane) {
  constexpr int CPL = Frag<DT>::kLaneBytes / 16;
  const int c0 = (lane >> 5) * CPL;
  if constexpr (DT == kBF16) {
    f.v[i] = tile[tile_chunk<DT>(key, c0 + i)];
  } else {
    u32x4 lo = tile[tile_chunk<DT>(key, c0 + 2 * i)], hi = tile[tile_chunk<DT>(key, c0 + 2 * i + 1)];
    f.v[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
}

// Candidate bookkeeping of one row (one wave): records are appended to a
// small LDS stage during a tile and flushed to the row's global buffer at the
// start of the next tile, so the tile-end wait for the next key tile never
// waits on fresh candidate stores.  State: cnt records in buf, nst in the
// stage, running threshold thr (records below it cannot be in the Top-K).
__device__ __forceinline__ int flush_stage(uint64_t* buf, int cnt, const uint64_t* stage, int nst, int lane) {
  for (int i = lane; i < nst; i += 64) buf[cnt + i] = stage[i];
  return cnt + nst;
}

struct Cut {
  int cnt;
  uint64_t thr;
};

// Cut the row's candidates (buffer + stage) back to between topk and `goal`
// records and raise the threshold to the cut's boundary; goal == topk keeps
// exactly the best topk, so the threshold becomes the K-th best record seen.
static __device__ __noinline__ Cut cut_candidates_d8(uint64_t* buf, int cnt, const uint64_t* stage, int nst,
                                                     uint32_t* hist, int topk, int goal, int lane) {
  cnt = flush_stage(buf, cnt, stage, nst, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  const SelectResult sel = select_records_d8(buf, cnt, (uint32_t)topk, hist, false, (uint32_t)goal, lane);
  return {compact_records_d8(buf, cnt, sel, lane), sel.prefix};
}

// Write the row's exact Top-K (min(topk, cnt) indices, then -1 padding).
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

// Key tile loaded straight from global memory into LDS (global_load_lds, 16
// bytes per lane, no staging registers): the KT keys of one 32 KiB tile,
// key-major with one pad chunk per key, 16-byte chunk c of tile key r at
// slot r * (CPR + 1) + c.  With that pitch the 16 lanes served together by
// a 16-byte LDS read (16 consecutive keys, one chunk) hit 16 different bank
// groups, and a lane's successive chunks sit at immediate offsets from one
// base address.  One load instruction fills 64 consecutive slots, i.e. about
// four consecutive key rows: the global reads are whole contiguous rows (a
// pad slot re-reads its row's last chunk).  Instruction n of a tile is
// issued by wave n % kWaves; the per-lane byte offsets are fixed, so a load
// costs no vector ALU work.  Completion: each wave waits for its own loads
// (vmcnt), then a workgroup barrier publishes the tile.
template <int DT>
struct DirectTile {
  static constexpr int RB = Frag<DT>::kRowBytes;
  static constexpr int CPR = RB / 16;                  // chunks per key
  static constexpr int KT = 32768 / RB;                // keys per tile: 128 bf16, 256 fp8
  static constexpr int SLOTS = KT * (CPR + 1);         // 2176 / 2304: whole instructions
  static constexpr int NI = SLOTS / 64;                // load instructions per tile
  static constexpr int PER_WAVE = (NI + kWaves - 1) / kWaves;
  static_assert(SLOTS % 64 == 0, "tile slots fill whole load instructions");
  const uint32_t* off;  // this wave's [PER_WAVE][64] source offsets (LDS), from the tile's first row
  int wave;             // wave-uniform

  // `table`: this wave's PER_WAVE x 64 LDS words (visible to the wave after
  // the next workgroup barrier).
  __device__ __forceinline__ void init(uint32_t* table, int wave_id, int lane) {
    wave = __builtin_amdgcn_readfirstlane(wave_id);
    off = table;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int p = 64 * (wave + kWaves * j) + lane;
      const int r = p / (CPR + 1), c = p % (CPR + 1);
      table[64 * j + lane] = (uint32_t)(r * RB + min(c, CPR - 1) * 16);
    }
  }
  // Issue this wave's loads of tile rows ts..ts+KT-1 into `slot` (keys at or
  // past N read key N-1, never scored: visibility masks them).
  __device__ __forceinline__ void load(u32x4* slot, const uint8_t* kbase, int ts, int N, int lane) const {
    if (ts + KT <= N) {
      const uint8_t* base = kbase + (size_t)ts * RB;
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int n = wave + kWaves * j;
        if (n < NI) __builtin_amdgcn_global_load_lds(base + off[64 * j + lane], slot + 64 * n, 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int n = wave + kWaves * j;
        if (n < NI) {
          const uint32_t o = off[64 * j + lane];
          const int key = min(ts + (int)(o / RB), N - 1);
          __builtin_amdgcn_global_load_lds(kbase + (size_t)key * RB + o % RB, slot + 64 * n, 16, 0, 0);
        }
      }
    }
  }
  // fp8 key scales of the tile's rows (4 bytes per lane, waves 0..KT/64-1).
  __device__ __forceinline__ void load_scales(float* kst, const float* kscb, int ts, int N, int lane) const {
    if (wave < KT / 64) {
      const int key = min(ts + 64 * wave + lane, N - 1);
      __builtin_amdgcn_global_load_lds(kscb + key, kst + 64 * wave, 4, 0, 0);
    }
  }
  // Fragment of tile key `key` (lane layout of load_frag).
  __device__ __forceinline__ static void frag(Frag<DT>& f, const u32x4* slot, int key, int lane) {
#pragma unroll
    for (int i = 0; i < Frag<DT>::kSteps; ++i) frag_step(f, slot, key, i, lane);
  }
  // k-step i of that fragment.
  __device__ __forceinline__ static void frag_step(Frag<DT>& f, const u32x4* slot, int key, int i, int lane) {
    constexpr int CPL = Frag<DT>::kLaneBytes / 16;
    const u32x4* row = slot + key * (CPR + 1) + (lane >> 5) * CPL;
    if constexpr (DT == kBF16) {
      f.v[i] = row[i];
    } else {
      const u32x4 lo = row[2 * i], hi = row[2 * i + 1];
      f.v[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
};
constexpr int kDirectSlots = 2304;  // max over dtypes of DirectTile::SLOTS

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
