// stream_common.h -- pieces shared by the streaming Top-K kernels (unpruned
// and pruned): LDS key tiles, per-row candidate bookkeeping, final emit.
#pragma once
#include <math.h>

#include "score_tile.h"
#include "select.h"

namespace dsa {


// Orders one wave's LDS accesses across its lanes (a value one lane stored
// is then visible to the others): a wavefront-scope fence plus a scheduling
// barrier.  No workgroup barrier is involved.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Orders a wave's global-memory accesses across its lanes: the candidate
// buffer of a row is written and read only by the row's wave, so a
// workgroup-scope fence suffices (the waves of a workgroup share one CU's
// vector L1, and this waits for the wave's stores); an agent-scope fence
// would also write back and invalidate the whole L2 of the XCD.
__device__ __forceinline__ void row_mem_sync() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup"); }

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
  row_mem_sync();
  const SelectResult sel = select_records_d8(buf, cnt, (uint32_t)topk, hist, false, (uint32_t)goal, lane);
  return {compact_records_d8(buf, cnt, sel, lane), sel.prefix};
}

// Write the row's exact Top-K (min(topk, cnt) indices, then -1 padding).
static __device__ __noinline__ void emit_topk_d8(uint64_t* buf, int cnt, const uint64_t* stage, int nst,
                                                 uint32_t* hist, int topk, int32_t* oi, float* os, int lane) {
  cnt = flush_stage(buf, cnt, stage, nst, lane);
  row_mem_sync();
  const int need = min(topk, cnt);
  SelectResult sel = {0, 0, 0};
  if (need > 0) sel = select_records_d8(buf, cnt, (uint32_t)need, hist, true, 0, lane);
  int base = 0;
  for (int i0 = 0; i0 < cnt; i0 += 512) {  // eight records per lane in flight
    uint64_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      r[j] = i < cnt ? buf[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      const bool keep = i < cnt && (r[j] & sel.mask) >= sel.prefix;
      const uint64_t bal = __ballot(keep);
      const uint32_t before =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (keep) {
        oi[base + before] = (int32_t)record_key(r[j]);
        if (os) os[base + before] = record_score(r[j]);
      }
      base += __popcll(bal);
    }
  }
  for (int j = need + lane; j < topk; j += 64) {
    oi[j] = -1;
    if (os) os[j] = -INFINITY;
  }
}

constexpr int kRaiseEvery = 32;  // kept records between threshold raises
constexpr int kCutGoal = 512;    // a forced cut keeps at most topk + kCutGoal records (a quarter of the spare room at most)

// Records a forced cut may keep: topk + min(kCutGoal, (cap - topk) / 4), so
// it frees at least three quarters of the room beyond topk.
__device__ __forceinline__ int cut_goal(int topk, int cap) { return topk + min(kCutGoal, (cap - topk) / 4); }

// Candidate state of one row (wave-uniform).  Besides the buffer (cnt
// records, nst more in the LDS stage) and the threshold thr, the row keeps a
// threshold histogram: 256 LDS bins over the score code c (the high half of
// a record), bin min(255, (c - base) >> shift), counting every kept record
// (the pruned kernel counts a record when it stages it, the streaming kernel
// when it flushes it, before any threshold raise reads the bins); base never
// exceeds the threshold's code, so every kept record lands in a bin.
struct RowState {
  uint64_t* buf;
  int cnt, nst;
  uint64_t thr;
  uint32_t base;
  int shift;
  int added;  // records kept since the last threshold raise
};

__device__ __forceinline__ uint32_t thr_bin(uint32_t code, uint32_t base, int shift) {
  return min(255u, (code - base) >> shift);
}

struct Rebuilt {
  int cnt;
  uint64_t thr;
  uint32_t base;
  int shift;
};

// Flush the stage, keep only the records >= thr; if more than `goal` remain,
// cut them by radix select to between topk and goal (the threshold becomes
// the cut's boundary); then rebuild the histogram over the kept records from
// base = the threshold's code, with a bin width that spans their codes.
static __device__ __noinline__ Rebuilt rebuild_candidates(uint64_t* buf, int cnt, const uint64_t* stage, int nst,
                                                          uint32_t* hist, uint64_t thr, int topk, int goal,
                                                          int lane) {
  cnt = flush_stage(buf, cnt, stage, nst, lane);
  row_mem_sync();
  cnt = compact_records_d8(buf, cnt, SelectResult{thr, ~0ull, 0u}, lane);
  if (cnt > goal) {
    row_mem_sync();
    const SelectResult sel = select_records_d8(buf, cnt, (uint32_t)topk, hist, false, (uint32_t)goal, lane);
    cnt = compact_records_d8(buf, cnt, sel, lane);
    thr = sel.prefix;
  }
  row_mem_sync();
  const uint32_t base = (uint32_t)(thr >> 32);
  uint32_t mx = base;
  for (int i = lane; i < cnt; i += 64) mx = max(mx, (uint32_t)(buf[i] >> 32));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d, 64));
  const uint32_t span = mx - base;
  const int shift = span ? max(0, 24 - (int)__builtin_clz(span)) : 0;  // span >> shift < 256
  for (int i = lane; i < 256; i += 64) hist[i] = 0u;
  for (int i = lane; i < cnt; i += 64) atomicAdd(&hist[thr_bin((uint32_t)(buf[i] >> 32), base, shift)], 1u);
  return {cnt, thr, base, shift};
}

__device__ __forceinline__ void apply_rebuild(RowState& rs, const Rebuilt& r) {
  rs.cnt = r.cnt;
  rs.nst = 0;
  rs.thr = r.thr;
  rs.base = r.base;
  rs.shift = r.shift;
  rs.added = kRaiseEvery;
}

// Inclusive prefix sum over the 64 lanes: row_shr DPP steps inside each row
// of 16 lanes, then the row totals read out and added to the later rows.
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t x, int lane) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int rw = lane >> 4;
  return (uint32_t)(v + (rw >= 1 ? r0 : 0) + (rw >= 2 ? r1 : 0) + (rw >= 3 ? r2 : 0));
}

// Raise the threshold to the lower edge of the highest bin b whose bins >= b
// hold at least topk records: at least topk kept records reach that code, so
// it is at most the K-th best record seen (and within one bin of it).  Lane l
// reads bins 252 - 4l .. 255 - 4l (the top bins in lane 0), so the records
// above a lane's bins are a prefix sum over the lanes before it.
__device__ __forceinline__ void raise_threshold(RowState& rs, const uint32_t* hist, int topk, int lane) {
  const u32x4 h = reinterpret_cast<const u32x4*>(hist)[63 - lane];  // h.w: bin 255 - 4 lane
  const uint32_t local = h.x + h.y + h.z + h.w;
  const uint32_t above = wave_prefix_incl(local, lane) - local;
  const uint64_t bal = __ballot(above < (uint32_t)topk && (uint32_t)topk <= above + local);
  rs.added = 0;
  if (!bal) return;  // fewer than topk records counted
  const int src = __builtin_ctzll(bal);
  uint32_t b = 4u * (63 - lane);
  if (above + h.w >= (uint32_t)topk)
    b += 3;
  else if (above + h.w + h.z >= (uint32_t)topk)
    b += 2;
  else if (above + h.w + h.z + h.y >= (uint32_t)topk)
    b += 1;
  b = (uint32_t)__builtin_amdgcn_readlane((int)b, src);
  const uint32_t code = rs.base + (b << rs.shift);
  if (code > (uint32_t)(rs.thr >> 32)) rs.thr = (uint64_t)code << 32;
}

// Key tile loaded straight from global memory into LDS (global_load_lds, 16
// bytes per lane, no staging registers): the KT keys of one tile of
// kTileBytes key bytes, shared by the kWaves waves of a workgroup,
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
template <int DT, int kTileBytes, int kWaves>
struct DirectTile {
  static constexpr int RB = Frag<DT>::kRowBytes;
  static constexpr int CPR = RB / 16;                  // chunks per key
  static constexpr int KT = kTileBytes / RB;           // keys per tile
  static constexpr int SLOTS = KT * (CPR + 1);         // LDS chunks, whole load instructions
  static constexpr int NI = SLOTS / 64;                // load instructions per tile
  static constexpr int PER_WAVE = (NI + kWaves - 1) / kWaves;
  static_assert(SLOTS % 64 == 0, "tile slots fill whole load instructions");
  static_assert(kWaves * (PER_WAVE - 1) <= NI, "only the last load of a wave may be past the tile");
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
  // past N read key N-1, never scored: visibility masks them).  All offsets
  // are read first (one LDS wait); every wave issues the first PER_WAVE - 1
  // instructions (8 (PER_WAVE - 1) <= NI), only the last one is guarded.
  __device__ __forceinline__ void load(u32x4* slot, const uint8_t* kbase, int ts, int N, int lane) const {
    uint32_t o[PER_WAVE];
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) o[j] = off[64 * j + lane];
    if (ts + KT <= N) {
      const uint8_t* base = kbase + (size_t)ts * RB;
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j)
        if (j < PER_WAVE - 1 || wave + kWaves * j < NI)
          __builtin_amdgcn_global_load_lds(base + o[j], slot + 64 * (wave + kWaves * j), 16, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j)
        if (j < PER_WAVE - 1 || wave + kWaves * j < NI) {
          const int key = min(ts + (int)(o[j] / RB), N - 1);
          __builtin_amdgcn_global_load_lds(kbase + (size_t)key * RB + o[j] % RB, slot + 64 * (wave + kWaves * j),
                                           16, 0, 0);
        }
    }
  }
  // One 4-byte word per tile row (fp8 key scale, key norm): dst[r] =
  // src[min(ts + r, N - 1)], 64 rows per instruction, instructions spread
  // over the waves.
  __device__ __forceinline__ void load_words(float* dst, const float* src, int ts, int N, int lane) const {
#pragma unroll
    for (int wr = 0; wr < KT / 64; wr += kWaves) {
      if (wr + wave < KT / 64) {
        const int key = min(ts + 64 * (wr + wave) + lane, N - 1);
        __builtin_amdgcn_global_load_lds(src + key, dst + 64 * (wr + wave), 4, 0, 0);
      }
    }
  }
  // 64 words of a per-key bitmap from the tile's first word on (the tile
  // uses the first KT / 32; indexes clamp to the last word), by the last wave.
  __device__ __forceinline__ void load_bits(uint32_t* dst, const uint32_t* bits, int ts, int words, int lane) const {
    if (wave == kWaves - 1)
      __builtin_amdgcn_global_load_lds(bits + min(ts / 32 + lane, words - 1), dst, 4, 0, 0);
  }
  // Fragment of tile key `key` (lane layout of load_frag).
  __device__ __forceinline__ static void frag(Frag<DT>& f, const u32x4* slot, int key, int lane) {
#pragma unroll
    for (int i = 0; i < Frag<DT>::kSteps; ++i) frag_step(f, slot, key, i, lane);
  }
  // k-step i of that fragment (the chunk order of load_frag).
  __device__ __forceinline__ static void frag_step(Frag<DT>& f, const u32x4* slot, int key, int i, int lane) {
    if constexpr (DT == kBF16) {
      const u32x4* row = slot + key * (CPR + 1) + (lane >> 5);
      f.v[i] = row[2 * i];
    } else {
      const u32x4* row = slot + key * (CPR + 1) + 2 * (lane >> 5);
      const u32x4 lo = row[4 * i], hi = row[4 * i + 1];
      f.v[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
};
// LDS chunks of a tile of `tile_bytes` key bytes, the larger over the dtypes
// (fp8: 9 chunks per 128-byte key).
constexpr int direct_slots(int tile_bytes) { return tile_bytes / 128 * 9; }

}  // namespace dsa
