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
//   workgroup = 4 waves = 8 consecutive query rows of one sequence,
//   wave      = 2 query rows held in registers as MFMA A fragments
//               (2 x 64 heads x 128 dims), plus their 64 head weights;
//   key tiles of 128 rows are staged in LDS (XOR-swizzled 16-byte chunks so
//   the 32-lane column reads are bank-conflict free) and shared by the
//   4 waves; every 32-key block feeds both rows of a wave.
//   After the head sum, lanes 0..31 hold row A's 32 scores and lanes 32..63
//   row B's, so the threshold test, ballot and append are one wave op.
//   Workgroups are issued longest-prefix first (causal imbalance).
#include <math.h>

#include "kernels.h"
#include "score_tile.h"
#include "select.h"

namespace dsa {

constexpr int kTileKeys = 128;
constexpr int kRowsPerWG = 8;

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

// Keep only records (r & mask) >= prefix, in place, preserving order.
__device__ __noinline__ int wave_compact(uint64_t* buf, int cnt, SelectResult sel, int lane) {
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
    const uint32_t before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (keep) buf[base + before] = r;
    base += __popcll(bal);
  }
  return base;
}

template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_topk_stream(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const float* __restrict__ qsc, const float* __restrict__ ksc, const int32_t* __restrict__ pos, int Q, int N,
    int topk, int cap, uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  constexpr int RB = Frag<DT>::kRowBytes;
  constexpr int CPR = RB / 16;
  constexpr int TILE_CHUNKS = kTileKeys * CPR;
  __shared__ u32x4 ktile[TILE_CHUNKS];
  __shared__ float kscale_tile[kTileKeys];
  __shared__ uint32_t hist[4][2048];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = gridDim.x - 1 - blockIdx.x;  // longest prefixes first
  const int b = blockIdx.y;
  const int tA = group * kRowsPerWG + 2 * wave, tB = tA + 1;
  const bool validA = tA < Q, validB = tB < Q;
  const size_t rowA = (size_t)b * Q + min(tA, Q - 1), rowB = (size_t)b * Q + min(tB, Q - 1);
  const int visA = validA ? min(max(pos[rowA] + 1, 0), N) : 0;
  const int visB = validB ? min(max(pos[rowB] + 1, 0), N) : 0;
  int wg_vis = 0;
  for (int j = 0; j < kRowsPerWG; ++j) {
    const int t = group * kRowsPerWG + j;
    if (t < Q) wg_vis = max(wg_vis, min(max(pos[(size_t)b * Q + t] + 1, 0), N));
  }
  const int wave_vis = max(visA, visB);

  QuerySide<DT> qa, qb;
  load_query<DT>(qa, q + rowA * kHeads * RB, w + rowA * kHeads, lane);
  load_query<DT>(qb, q + rowB * kHeads * RB, w + rowB * kHeads, lane);
  const float qscale = (DT == kFP8) ? qsc[(lane < 32) ? rowA : rowB] : 1.0f;

  const bool hiHalf = lane >= 32;
  const int myVis = hiHalf ? visB : visA;
  uint64_t* bufA = cand + rowA * (size_t)cap;
  uint64_t* bufB = cand + rowB * (size_t)cap;
  int cntA = 0, cntB = 0;
  uint64_t thrA = 0, thrB = 0;
  uint32_t* my_hist = hist[wave];
  const uint8_t* kbase = k + (size_t)b * N * RB;

  for (int ts = 0; ts < wg_vis; ts += kTileKeys) {
    __syncthreads();
    for (int c = tid; c < TILE_CHUNKS; c += 256) {
      const int key = c / CPR, ch = c % CPR;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ts + key < N) v = *reinterpret_cast<const u32x4*>(kbase + (size_t)(ts + key) * RB + ch * 16);
      ktile[swz_chunk<DT>(key, ch)] = v;
    }
    if constexpr (DT == kFP8) {
      if (tid < kTileKeys) kscale_tile[tid] = (ts + tid < N) ? ksc[(size_t)b * N + ts + tid] : 1.0f;
    }
    __syncthreads();
    for (int sub = 0; sub < kTileKeys; sub += 32) {
      const int kb = ts + sub;
      if (kb >= wave_vis) break;  // wave-uniform
      Frag<DT> f;
      load_frag_lds<DT>(f, ktile, sub + (lane & 31), lane);
      const float pA = query_partial<DT>(qa, f);
      const float pB = query_partial<DT>(qb, f);
      float s = combine_halves(pA, pB, lane);
      if constexpr (DT == kFP8) s = apply_scales(s, qscale, kscale_tile[sub + (lane & 31)]);
      const int key = kb + (lane & 31);
      const uint64_t rec = make_record(s, (uint32_t)key);
      const uint64_t thr = hiHalf ? thrB : thrA;
      bool pass = key < myVis && rec >= thr;
      uint64_t bal = __ballot(pass);
      int nA = __popcll(bal & 0xFFFFFFFFull), nB = __popcll(bal >> 32);
      if (cntA + nA > cap) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
        SelectResult sel = wave_radix_select(bufA, cntA, topk, my_hist, lane);
        cntA = wave_compact(bufA, cntA, sel, lane);
        thrA = sel.prefix & sel.mask;
      }
      if (cntB + nB > cap) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
        SelectResult sel = wave_radix_select(bufB, cntB, topk, my_hist, lane);
        cntB = wave_compact(bufB, cntB, sel, lane);
        thrB = sel.prefix & sel.mask;
      }
      pass = key < myVis && rec >= (hiHalf ? thrB : thrA);
      bal = __ballot(pass);
      nA = __popcll(bal & 0xFFFFFFFFull);
      nB = __popcll(bal >> 32);
      const uint32_t before =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (pass) {
        if (hiHalf)
          bufB[cntB + (before - nA)] = rec;
        else
          bufA[cntA + before] = rec;
      }
      cntA += nA;
      cntB += nB;
    }
  }

  // final exact selection of each row's min(topk, visible) best records
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  for (int h = 0; h < 2; ++h) {
    const bool valid = h ? validB : validA;
    if (!valid) continue;
    const size_t row = h ? rowB : rowA;
    uint64_t* buf = h ? bufB : bufA;
    const int cnt = h ? cntB : cntA;
    const int need = min(topk, cnt);
    SelectResult sel = {0, 0};
    if (need > 0) sel = wave_radix_select(buf, cnt, need, my_hist, lane);
    int32_t* oi = out_idx + row * (size_t)topk;
    float* os = out_score ? out_score + row * (size_t)topk : nullptr;
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
}

hipError_t launch_topk_stream(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx,
                              float* out_score, hipStream_t st) {
  dim3 grid((p.Q + kRowsPerWG - 1) / kRowsPerWG, p.B);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_topk_stream<kBF16>, grid, dim3(256), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, topk, cap, cand, out_idx, out_score);
  else
    hipLaunchKernelGGL(k_topk_stream<kFP8>, grid, dim3(256), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       p.Q, p.N, topk, cap, cand, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace dsa
