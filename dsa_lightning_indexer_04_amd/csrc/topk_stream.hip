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
