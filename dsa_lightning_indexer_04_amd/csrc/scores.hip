// scores.hip -- full score rows and exact selection over stored score rows.
//
// k_scores: one wave per (query row, 32-key block), keys read straight from
// HBM into MFMA fragments (each key is used by one query here, so staging it
// through LDS would buy nothing).  Used for the score-matrix entry point and,
// for few query rows (decode: one row per sequence against a long key cache,
// DeepSeek DSA FLOPs notes, indexer "Decode" section), as the split-N first
// half of the Top-K: the rows are [B*Q, N] floats, tiny next to the keys.
//
// k_select_rows: one workgroup per row, radix select over the row's records
// (score code, inverted key index) -> the min(k, visible) best keys.
#include <math.h>

#include "kernels.h"
#include "score_tile.h"

namespace dsa {

template <int DT>
__global__ __launch_bounds__(256) void k_scores(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                                                const float* __restrict__ w, const float* __restrict__ qsc,
                                                const float* __restrict__ ksc, const int32_t* __restrict__ pos,
                                                float* __restrict__ out, int Q, int N, int keys_per_wg) {
  constexpr int RB = Frag<DT>::kRowBytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t row = blockIdx.x;  // b * Q + t
  const int b = (int)(row / (size_t)Q);
  const int vis = min(max(pos[row] + 1, 0), N);
  const int k0 = blockIdx.y * keys_per_wg;
  const int k1 = min(N, k0 + keys_per_wg);
  float* orow = out + row * (size_t)N;
  const uint8_t* kbase = k + (size_t)b * N * RB;
  const float qscale = (DT == kFP8) ? qsc[row] : 1.0f;

  QuerySide<DT> qs;
  load_query<DT>(qs, q + row * kHeads * RB, w + row * kHeads, lane);
  for (int kb = k0 + 32 * wave; kb < k1; kb += 128) {
    const int key = kb + (lane & 31);
    float s = -INFINITY;
    if (kb < vis) {  // wave-uniform
      const int kl = min(key, N - 1);
      Frag<DT> f;
      load_frag<DT>(f, kbase + (size_t)kl * RB, lane);
      const float part = query_partial<DT>(qs, f);
      float tot = combine_single(part);
      if constexpr (DT == kFP8) tot = apply_scales(tot, qscale, ksc[(size_t)b * N + kl]);
      s = key < vis ? tot : -INFINITY;
    }
    if (lane < 32 && key < k1) orow[key] = s;
  }
}

hipError_t launch_scores(const Problem& p, float* scores, hipStream_t st) {
  const int prof_slot = prof_open("k_scores", st);
  const int kpw = 2048;
  dim3 grid((unsigned)(p.B * p.Q), (p.N + kpw - 1) / kpw);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_scores<kBF16>, grid, dim3(256), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       scores, p.Q, p.N, kpw);
  else
    hipLaunchKernelGGL(k_scores<kFP8>, grid, dim3(256), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       scores, p.Q, p.N, kpw);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- row select

__device__ __forceinline__ uint64_t row_record(const float* srow, int i) { return make_record(srow[i], (uint32_t)i); }

__global__ __launch_bounds__(1024) void k_select_rows(const float* __restrict__ scores, const int32_t* __restrict__ pos,
                                                      int N, int topk, int32_t* __restrict__ out_idx,
                                                      float* __restrict__ out_score) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wave_tot[16];
  __shared__ uint32_t sel_bin, sel_above, sel_count;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const size_t row = blockIdx.x;
  const int vis = min(max(pos[row] + 1, 0), N);
  const int need = min(topk, vis);
  const float* srow = scores + row * (size_t)N;
  int32_t* oi = out_idx + row * (size_t)topk;
  float* os = out_score ? out_score + row * (size_t)topk : nullptr;

  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)need;
  if (need > 0) {
    for (int pass = 0; pass < 6; ++pass) {
      const int S = (pass == 0) ? 53 : (pass == 1) ? 42 : (pass == 2) ? 32 : (pass == 3) ? 21 : (pass == 4) ? 10 : 0;
      const int W = (pass == 2 || pass == 5) ? 10 : 11;
      const uint32_t nb = 1u << W;
      for (uint32_t i = tid; i < nb; i += blockDim.x) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < vis; i += blockDim.x) {
        uint64_t r = row_record(srow, i);
        if ((r & mask) == prefix) atomicAdd(&hist[(uint32_t)(r >> S) & (nb - 1)], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        const uint32_t bpl = nb / 64;
        uint32_t local = 0;
        for (uint32_t j = 0; j < bpl; ++j) local += hist[lane * bpl + j];
        uint32_t incl = local;
        for (int d = 1; d < 64; d <<= 1) {
          uint32_t y = __shfl_down(incl, d, 64);
          if (lane + d < 64) incl += y;
        }
        const uint32_t above = incl - local;
        const bool mine = above < remaining && remaining <= above + local;
        if (mine) {
          uint32_t acc = above;
          for (int j = (int)bpl - 1; j >= 0; --j) {
            uint32_t h = hist[lane * bpl + j];
            if (acc + h >= remaining) {
              sel_bin = lane * bpl + j;
              sel_above = acc;
              sel_count = h;
              break;
            }
            acc += h;
          }
        }
      }
      __syncthreads();
      prefix |= (uint64_t)sel_bin << S;
      mask |= (uint64_t)(nb - 1) << S;
      remaining -= sel_above;
      const bool done = (sel_count == remaining);
      __syncthreads();
      if (done) break;
    }
  }
  // deterministic compaction in key order
  uint32_t base = 0;
  for (int i0 = 0; i0 < vis; i0 += blockDim.x) {
    const int i = i0 + tid;
    bool keep = false;
    uint64_t r = 0;
    if (i < vis) {
      r = row_record(srow, i);
      keep = (r & mask) >= prefix;
    }
    const uint64_t bal = __ballot(keep);
    const uint32_t before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (lane == 0) wave_tot[wave] = __popcll(bal);
    __syncthreads();
    uint32_t off = base;
    for (int v = 0; v < wave; ++v) off += wave_tot[v];
    uint32_t tot = 0;
    for (int v = 0; v < nw; ++v) tot += wave_tot[v];
    if (keep) {
      oi[off + before] = (int32_t)i;
      if (os) os[off + before] = record_score(r);
    }
    base += tot;
    __syncthreads();
  }
  for (int j = need + tid; j < topk; j += blockDim.x) {
    oi[j] = -1;
    if (os) os[j] = -INFINITY;
  }
}

hipError_t launch_select_rows(const Problem& p, const float* scores, int topk, int32_t* out_idx, float* out_score,
                              hipStream_t st) {
  const int prof_slot = prof_open("k_select_rows", st);
  hipLaunchKernelGGL(k_select_rows, dim3(p.B * p.Q), dim3(1024), 0, st, scores, p.pos, p.N, topk, out_idx,
                     out_score);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

}  // namespace dsa
