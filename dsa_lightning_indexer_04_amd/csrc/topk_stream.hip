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
#include "stream_common.h"

namespace dsa {

template <int DT>
struct BlockAcc {
  f32x16 s0, s1;  // heads 0..31 / 32..63 of one query against 32 keys
};

// Candidate state of one row (one wave): cnt records in the global buffer,
// nst in the LDS stage, running threshold thr and its float floor thr_f.
struct Cands {
  int cnt, nst;
  uint64_t thr;
  float thr_f;
};

// Append the records of one scored 32-key block (lanes 0..31; `live` masks
// keys that are not visible or not real).  The stage has room: the caller
// flushes it and cuts the buffer at tile boundaries.
__device__ __forceinline__ void append_block(Cands& c, float s, int key, bool live, uint64_t* stage, uint32_t* hist,
                                             int lane) {
  if (__ballot(live && s >= c.thr_f)) {  // cheap float pre-test; rare once thr has risen
    const uint64_t rec = make_record(s, (uint32_t)key);
    const bool take = live && rec >= c.thr;
    const uint64_t bal = __ballot(take);
    if (take) {
      stage[c.nst + __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)] = rec;
      atomicAdd(&hist[(uint32_t)(rec >> kH1Shift)], 1u);
    }
    c.nst += __popcll(bal);
  }
}

// Flush the stage to the buffer; if `room` more records could overflow the
// buffer, cut it back (radix select) and raise the threshold.
__device__ __forceinline__ void flush_and_cut(Cands& c, uint64_t* buf, const uint64_t* stage, uint32_t* hist,
                                              int topk, int cap, int room, int lane) {
  if (c.nst) {
    c.cnt = flush_stage(buf, c.cnt, stage, c.nst, lane);
    c.nst = 0;
  }
  if (c.cnt > cap - room) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
    const SelectResult sel =
        select_records(buf, c.cnt, (uint32_t)topk, hist, false, (uint32_t)(topk + (cap - topk) / 2), lane);
    c.cnt = compact_records(buf, c.cnt, sel, hist, lane);
    c.thr = sel.prefix;
    c.thr_f = record_floor(c.thr);
  }
}

template <int DT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_topk_stream(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ qsc, const float* __restrict__ ksc, const int32_t* __restrict__ pos, int Q, int N,
    int topk, int cap, uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  constexpr int RB = Frag<DT>::kRowBytes;
  constexpr int KT = kTileBytes / RB;  // keys per tile
  constexpr int NSB = KT / 32;         // 32-key blocks per tile (even)
  __shared__ u32x4 ktile[2][kTileChunks];
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
  Cands cs{0, 0, 0, -INFINITY};
  const uint8_t* kbase = k + (size_t)b * N * RB;
  const float* kscb = (DT == kFP8) ? ksc + (size_t)b * N : nullptr;

  TileFetch<DT> tf;
  const int ntiles = (wg_vis + KT - 1) / KT;
  if (ntiles > 0) {
    tf.fetch(kbase, kscb, 0, N, tid);
    tf.commit(ktile[0], kscale_tile[0], tid);
  }
  wait_vmem_all();
  __syncthreads();

  // Software pipeline over 32-key blocks j = 0, 1, ...: step j issues block
  // j's MFMAs (key fragment from the LDS tile) interleaved with the head sum
  // of block j-1 (from registers), then appends block j-1.  Every step runs
  // the same straight-line code; keys past the row's visible prefix and the
  // empty block -1 are masked at the append.  acc[j & 1] holds block j,
  // kscl[j & 1] its fp8 key scales.
  BlockAcc<DT> acc[2];
  acc[0].s0 = acc[0].s1 = acc[1].s0 = acc[1].s1 = zero16();
  float kscl[2] = {1.0f, 1.0f};
  const int lk = lane & 31;
  for (int ti = 0; ti < ntiles; ++ti) {
    const int cur = ti & 1;
    flush_and_cut(cs, buf, my_stage, my_hist, topk, cap, KT, lane);
    if (ti + 1 < ntiles) tf.fetch(kbase, kscb, (ti + 1) * KT, N, tid);
#pragma unroll
    for (int sub = 0; sub < NSB; ++sub) {
      const int j = ti * NSB + sub;
      BlockAcc<DT>& an = acc[sub & 1];
      const BlockAcc<DT>& ap = acc[(sub & 1) ^ 1];
      Frag<DT> f;
      load_frag_lds<DT>(f, ktile[cur], 32 * sub + lk, lane);
      float s = combine_single(pipelined_partial<DT>(qs, f, ap.s0, ap.s1, an.s0, an.s1));
      if constexpr (DT == kFP8) {
        s = apply_scales(s, qscale, kscl[(sub & 1) ^ 1]);
        kscl[sub & 1] = kscale_tile[cur][32 * sub + lk];
      }
      const int key = 32 * (j - 1) + lk;
      append_block(cs, s, key, lane < 32 && j > 0 && key < vis, my_stage, my_hist, lane);
    }
    if (ti + 1 < ntiles) tf.commit(ktile[cur ^ 1], kscale_tile[cur ^ 1], tid);
    __syncthreads();
  }
  if (!valid) return;
  if (ntiles > 0) {  // drain: the last block, j = ntiles * NSB - 1, is in acc[1]
    flush_and_cut(cs, buf, my_stage, my_hist, topk, cap, 32, lane);
    float s = combine_single(head_partial(acc[1].s0, acc[1].s1, qs.wl));
    if constexpr (DT == kFP8) s = apply_scales(s, qscale, kscl[1]);
    const int key = 32 * (ntiles * NSB - 1) + lk;
    append_block(cs, s, key, lane < 32 && key < vis, my_stage, my_hist, lane);
  }
  emit_topk(buf, cs.cnt, my_stage, cs.nst, my_hist, topk, out_idx + row * (size_t)topk,
            out_score ? out_score + row * (size_t)topk : nullptr, lane);
}

hipError_t launch_topk_stream(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx,
                              float* out_score, hipStream_t st) {
  const int prof_slot = prof_open("k_topk_stream", st);
  dim3 grid((p.Q + kWaves - 1) / kWaves, p.B);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_topk_stream<kBF16>, grid, dim3(kWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, topk, cap, cand, out_idx, out_score);
  else
    hipLaunchKernelGGL(k_topk_stream<kFP8>, grid, dim3(kWaves * 64), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, topk, cap, cand, out_idx, out_score);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

}  // namespace dsa
