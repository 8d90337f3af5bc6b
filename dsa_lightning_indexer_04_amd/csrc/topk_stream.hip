// topk_stream.hip -- fused scoring + exact streaming Top-K for prefill blocks.
//
// The indexer must score the whole causal prefix of every query before it
// knows its Top-K (DeepSeek DSA FLOPs notes, remark at the end of
// "Full-prefix index scoring"); this kernel does that without ever storing
// the score matrix.  Each row keeps a running threshold and a candidate
// buffer of records in global memory; a key is appended only if its record
// is not below the threshold, and when the buffer fills it is cut back to the
// row's best `topk` by radix select, which also raises the threshold.  At the
// end the buffer's best min(topk, visible) records are the exact Top-K.
//
// Organisation (gfx950):
//   workgroup = 8 waves = 8 consecutive query rows of one sequence, one row
//               per wave held in registers as MFMA A fragments (64 heads x
//               128 dims) plus its head weights; two waves per SIMD, so one
//               wave's MFMAs overlap the other's fp32 epilogue;
//   key tiles (16 KiB: 64 bf16 or 128 fp8 keys) are double-buffered in LDS:
//   the next tile is fetched into registers while the current one is scored
//   and stored at the tile's end, in an XOR-swizzled chunk order so the
//   32-lane column reads are bank-conflict free; all 8 waves read each tile.
//   After the head sum every lane holds the score of key l%32, so the
//   threshold test, ballot and append are one wave op on lanes 0..31.
//   Workgroups are issued longest-prefix first (causal imbalance).
#include <math.h>

#include "kernels.h"
#include "score_tile.h"
#include "select.h"

namespace dsa {

constexpr int kWaves = 8;           // query rows per workgroup, one per wave
constexpr int kTileBytes = 16384;   // one LDS key tile (64 bf16 or 128 fp8 keys)

template <int DT>
__device__ __forceinline__ int swz_chunk(int key, int c) {
  constexpr int CPR = Frag<DT>::kRowBytes / 16;  // 16-byte chunks per row
  return key * CPR + (c ^ (key & (CPR - 1)));
}

// Fragment of key `key` (tile-relative) from the swizzled LDS tile.
template <int DT>
__device__ __forceinline__ void load_frag_lds(Frag<DT>& f, const u32x4* tile, int key, int lane) {
  constexpr int CPL = Frag<DT>::kLaneBytes / 16;  // chunks per lane
  const int c0 = (lane >> 5) * CPL;
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = tile[swz_chunk<DT>(key, c0 + i)];
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 lo = tile[swz_chunk<DT>(key, c0 + 2 * i)], hi = tile[swz_chunk<DT>(key, c0 + 2 * i + 1)];
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

// Cut the row's candidates (buffer + stage) back towards `topk` and raise
// the threshold.  Rare: called when the buffer would overflow.
__device__ __noinline__ Cut cut_candidates(uint64_t* buf, int cnt, const uint64_t* stage, int nst, uint32_t* hist,
                                           int topk, int cap, int lane) {
  cnt = flush_stage(buf, cnt, stage, nst, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  const SelectResult sel =
      select_records(buf, cnt, (uint32_t)topk, hist, false, (uint32_t)(topk + (cap - topk) / 2), lane);
  return {compact_records(buf, cnt, sel, hist, lane), sel.prefix};
}

// Write the row's exact Top-K (min(topk, cnt) indices, then -1 padding).
__device__ __noinline__ void emit_topk(uint64_t* buf, int cnt, const uint64_t* stage, int nst, uint32_t* hist,
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
  float ks;

  __device__ __forceinline__ void fetch(const uint8_t* kbase, const float* kscb, int ts, int N, int tid) {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * kWaves * 64;
      const int key = c / CPR, ch = c % CPR;
      const int gk = min(ts + key, N - 1);
      v[j] = *reinterpret_cast<const u32x4*>(kbase + (size_t)gk * Frag<DT>::kRowBytes + ch * 16);
    }
    if constexpr (DT == kFP8) {
      if (tid < KT) ks = kscb[min(ts + tid, N - 1)];
    }
  }
  __device__ __forceinline__ void commit(u32x4* tile, float* kst, int tid) const {
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int c = tid + j * kWaves * 64;
      tile[swz_chunk<DT>(c / CPR, c % CPR)] = v[j];
    }
    if constexpr (DT == kFP8) {
      if (tid < KT) kst[tid] = ks;
    }
  }
};

template <int DT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_topk_stream(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ qsc, const float* __restrict__ ksc, const int32_t* __restrict__ pos, int Q, int N,
    int topk, int cap, uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  constexpr int RB = Frag<DT>::kRowBytes;
  constexpr int KT = kTileBytes / RB;  // keys per tile
  __shared__ u32x4 ktile[2][kTileBytes / 16];
  __shared__ float kscale_tile[2][KT];
  __shared__ uint32_t hist[kWaves][kH1Bins];
  __shared__ uint64_t stage[kWaves][KT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = gridDim.x - 1 - blockIdx.x;  // longest prefixes first
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

  QuerySide<DT> qs;
  load_query<DT>(qs, q + row * kHeads * RB, w + row * kHeads, lane);
  const float qscale = (DT == kFP8) ? qsc[row] : 1.0f;

  uint32_t* my_hist = hist[wave];
  uint64_t* my_stage = stage[wave];
  for (uint32_t i = lane; i < kH1Bins; i += 64) my_hist[i] = 0;
  uint64_t* buf = cand + row * (size_t)cap;
  int cnt = 0, nst = 0;
  uint64_t thr = 0;
  const uint8_t* kbase = k + (size_t)b * N * RB;
  const float* kscb = (DT == kFP8) ? ksc + (size_t)b * N : nullptr;

  TileFetch<DT> tf;
  const int ntiles = (wg_vis + KT - 1) / KT;
  if (ntiles > 0) {
    tf.fetch(kbase, kscb, 0, N, tid);
    tf.commit(ktile[0], kscale_tile[0], tid);
  }
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const int cur = ti & 1;
    const int ts = ti * KT;
    if (nst) {
      cnt = flush_stage(buf, cnt, my_stage, nst, lane);
      nst = 0;
    }
    if (ti + 1 < ntiles) tf.fetch(kbase, kscb, ts + KT, N, tid);
#pragma unroll
    for (int sub = 0; sub < KT; sub += 32) {
      const int kb = ts + sub;
      if (kb < vis) {  // wave-uniform
        Frag<DT> f;
        load_frag_lds<DT>(f, ktile[cur], sub + (lane & 31), lane);
        float s = combine_single(query_partial<DT>(qs, f));
        if constexpr (DT == kFP8) s = apply_scales(s, qscale, kscale_tile[cur][sub + (lane & 31)]);
        const int key = kb + (lane & 31);
        const uint64_t rec = make_record(s, (uint32_t)key);
        const bool live = lane < 32 && key < vis;
        uint64_t bal = __ballot(live && rec >= thr);
        if (bal) {
          if (cnt + nst + __popcll(bal) > cap) {
            const Cut c = cut_candidates(buf, cnt, my_stage, nst, my_hist, topk, cap, lane);
            cnt = c.cnt;
            thr = c.thr;
            nst = 0;
            bal = __ballot(live && rec >= thr);
          }
          if (live && rec >= thr) {
            my_stage[nst + __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)] = rec;
            atomicAdd(&my_hist[(uint32_t)(rec >> kH1Shift)], 1u);
          }
          nst += __popcll(bal);
        }
      }
    }
    if (ti + 1 < ntiles) tf.commit(ktile[cur ^ 1], kscale_tile[cur ^ 1], tid);
    __syncthreads();
  }
  if (!valid) return;
  emit_topk(buf, cnt, my_stage, nst, my_hist, topk, out_idx + row * (size_t)topk,
            out_score ? out_score + row * (size_t)topk : nullptr, lane);
}

hipError_t launch_topk_stream(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx,
                              float* out_score, hipStream_t st) {
  dim3 grid((p.Q + kWaves - 1) / kWaves, p.B);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_topk_stream<kBF16>, grid, dim3(kWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, topk, cap, cand, out_idx, out_score);
  else
    hipLaunchKernelGGL(k_topk_stream<kFP8>, grid, dim3(kWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, topk, cap, cand, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace dsa
