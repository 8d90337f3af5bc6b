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

constexpr int kDepth = 2;  // key blocks per wave in flight (k_scores)

template <int DT>
__global__ __launch_bounds__(256) void k_scores(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                                                const float* __restrict__ w, const float* __restrict__ qsc,
                                                const float* __restrict__ ksc, const int32_t* __restrict__ pos,
                                                float* __restrict__ out, uint32_t* __restrict__ row_hist, int Q,
                                                int N, int keys_per_wg) {
  // With row_hist: the workgroup's share of its row's code histogram, in
  // four LDS copies (lane & 3) so that a wave's adds to one bin spread out.
  __shared__ uint32_t lhist[4][kRowHistBins];
  if (row_hist) {  // kernel-uniform
    for (int i = threadIdx.x; i < 4 * kRowHistBins; i += blockDim.x) (&lhist[0][0])[i] = 0u;
    __syncthreads();
  }
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
  // Keys stream straight from HBM: a wave scores the 32-key blocks k0 +
  // 32 wave + 128 m, m = 0, 1, ..., with the next kDepth - 1 of them already
  // loading into a ring of fragments.  The prefetch is unconditional (a block
  // past the end reads key N - 1), which keeps the number of loads in flight
  // fixed for the waits.
  const int lk = lane & 31;
  Frag<DT> f[kDepth];
  int kb = k0 + 32 * wave;
#pragma unroll
  for (int h = 0; h < kDepth - 1; ++h) load_frag<DT>(f[h], kbase + (size_t)min(kb + 128 * h + lk, N - 1) * RB, lane);
  for (; kb < k1; kb += 128 * kDepth) {
#pragma unroll
    for (int h = 0; h < kDepth; ++h) {
      const int kc = kb + 128 * h;  // this block
      load_frag<DT>(f[(h + kDepth - 1) % kDepth], kbase + (size_t)min(kc + 128 * (kDepth - 1) + lk, N - 1) * RB, lane);
      if (kc < k1) {
        const int key = kc + lk;
        float s = -INFINITY;
        if (kc < vis) {  // wave-uniform
          float tot = combine_swap(query_partial<DT>(qs, f[h]));
          if constexpr (DT == kFP8) tot = apply_scales(tot, qscale, ksc[(size_t)b * N + min(key, N - 1)]);
          s = key < vis ? tot : -INFINITY;
        }
        if (lane < 32 && key < k1) {
          orow[key] = s;
          if (row_hist && key < vis) atomicAdd(&lhist[lane & 3][mono_code(s) >> 21], 1u);
        }
      }
    }
  }
  if (row_hist) {
    __syncthreads();
    for (int i = threadIdx.x; i < kRowHistBins; i += blockDim.x) {
      const uint32_t c = lhist[0][i] + lhist[1][i] + lhist[2][i] + lhist[3][i];
      if (c) atomicAdd(&row_hist[row * kRowHistBins + i], c);
    }
  }
}

__global__ void k_zero_words(uint32_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_scores(const Problem& p, float* scores, uint32_t* row_hist, hipStream_t st) {
  if (row_hist) {  // a fill kernel, not a memset: the launch may be captured into a graph
    const size_t n = (size_t)p.B * p.Q * kRowHistBins;
    hipLaunchKernelGGL(k_zero_words, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, row_hist, n);
  }
  const int prof_slot = prof_open("k_scores", st);
  const int kpw = 8192;  // keys per workgroup: long streams amortise the query load
  dim3 grid((unsigned)(p.B * p.Q), (p.N + kpw - 1) / kpw);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_scores<kBF16>, grid, dim3(256), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       scores, row_hist, p.Q, p.N, kpw);
  else
    hipLaunchKernelGGL(k_scores<kFP8>, grid, dim3(256), 0, st, p.q, p.k, p.w, p.q_scale, p.k_scale, p.pos,
                       scores, row_hist, p.Q, p.N, kpw);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- row select

__device__ __forceinline__ uint64_t row_record(const float* srow, int i) { return make_record(srow[i], (uint32_t)i); }

constexpr int kSelCand = 8192;  // records kept in LDS after the first pass

// Slots for the kept elements of one wave-wide step: one LDS atomic add per
// wave reserves a contiguous run (slot order across waves is unspecified).
__device__ __forceinline__ uint32_t wave_reserve(bool keep, uint32_t* counter, int lane) {
  const uint64_t bal = __ballot(keep);
  const uint32_t before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
  uint32_t base = 0;
  if (lane == 0 && bal) base = atomicAdd(counter, (uint32_t)__popcll(bal));
  return __shfl(base, 0, 64) + before;
}

// Visit the records of row[0..cnt) (score, key index): 16 scores per thread
// per round, as four 16-byte loads when the row is 16-byte aligned (cnt
// rounded down to a multiple of 4; the tail and unaligned rows go scalar),
// so a workgroup keeps 64 KB of reads in flight.
template <typename F>
__device__ __forceinline__ void for_row_records(const float* srow, int cnt, bool aligned, int tid, int nthreads,
                                                F&& f) {
  int done = 0;
  if (aligned) {
    const int n4 = cnt / 4;
    const float4* s4 = reinterpret_cast<const float4*>(srow);
    for (int j0 = 0; j0 < n4; j0 += 4 * nthreads) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * nthreads + tid;
        v[u] = j < n4 ? s4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * nthreads + tid;
        const bool ok = j < n4;
        f(ok, make_record(v[u].x, (uint32_t)(4 * j + 0)));
        f(ok, make_record(v[u].y, (uint32_t)(4 * j + 1)));
        f(ok, make_record(v[u].z, (uint32_t)(4 * j + 2)));
        f(ok, make_record(v[u].w, (uint32_t)(4 * j + 3)));
      }
    }
    done = 4 * n4;
  }
  for (int i0 = done; i0 < cnt; i0 += nthreads) {
    const int i = i0 + tid;
    const bool ok = i < cnt;
    f(ok, ok ? row_record(srow, i) : 0ull);
  }
}

// One workgroup per row.  Radix select over the row's records with 11/11/10-
// bit digits; after the first pass, if the records at or above the boundary
// bin fit, they move to LDS and later passes and the output read them there
// instead of the row.  The order of the selected keys within the output row
// is unspecified.
__global__ __launch_bounds__(1024) void k_select_rows(const float* __restrict__ scores,
                                                      const uint32_t* __restrict__ row_hist,
                                                      const int32_t* __restrict__ pos, int N, int topk,
                                                      int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  // 8 copies of the histogram (lane & 7 picks one): a row's scores share
  // their leading bits, so most records fall into a few bins, and one copy
  // would serialise a wave's 64 atomic adds on the same address.
  __shared__ uint32_t hist[8][2048];
  __shared__ uint64_t cand[kSelCand];
  __shared__ uint32_t sel_bin, sel_above, sel_count, fill;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = blockIdx.x;
  const int vis = min(max(pos[row] + 1, 0), N);
  const int need = min(topk, vis);
  const float* srow = scores + row * (size_t)N;
  int32_t* oi = out_idx + row * (size_t)topk;
  float* os = out_score ? out_score + row * (size_t)topk : nullptr;

  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)need;
  int ncand = -1;  // < 0: records are read from the row
  const bool aligned = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  if (need > 0) {
    for (int pass = 0; pass < 6; ++pass) {
      const int S = (pass == 0) ? 53 : (pass == 1) ? 42 : (pass == 2) ? 32 : (pass == 3) ? 21 : (pass == 4) ? 10 : 0;
      const int W = (pass == 2 || pass == 5) ? 10 : 11;
      const uint32_t nb = 1u << W;
      // the first digit's histogram may come with the rows (row_hist): the
      // same counts, without a pass over the row
      const bool given = pass == 0 && row_hist != nullptr;
      for (uint32_t i = tid; i < 8 * nb; i += blockDim.x)
        hist[i / nb][i % nb] = (given && i < nb) ? row_hist[row * kRowHistBins + i] : 0u;
      __syncthreads();
      auto add = [&](bool ok, uint64_t r) {
        if (ok && (r & mask) == prefix) atomicAdd(&hist[lane & 7][(uint32_t)(r >> S) & (nb - 1)], 1u);
      };
      if (given) {
      } else if (ncand < 0) {
        for_row_records(srow, vis, aligned, tid, (int)blockDim.x, add);
      } else {
        for (int i = tid; i < ncand; i += blockDim.x) add(true, cand[i]);
      }
      __syncthreads();
      for (uint32_t i = tid; i < nb; i += blockDim.x) {  // fold the copies into copy 0
        uint32_t t = hist[0][i];
#pragma unroll
        for (int c = 1; c < 8; ++c) t += hist[c][i];
        hist[0][i] = t;
      }
      __syncthreads();
      if (wave == 0) {
        const uint32_t bpl = nb / 64;
        uint32_t local = 0;
        for (uint32_t j = 0; j < bpl; ++j) local += hist[0][lane * bpl + j];
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
            uint32_t h = hist[0][lane * bpl + j];
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
      const uint32_t count = sel_count;
      const bool done = (count == remaining);
      const uint32_t kept_total = (uint32_t)need - remaining + count;  // records with (r & mask) >= prefix
      __syncthreads();
      if (done) break;
      if (ncand < 0 && kept_total <= (uint32_t)kSelCand) {
        // the candidates (bins at or above the boundary) move to LDS, key order
        if (tid == 0) fill = 0;
        __syncthreads();
        for_row_records(srow, vis, aligned, tid, (int)blockDim.x, [&](bool ok, uint64_t r) {
          const bool keep = ok && (r & mask) >= prefix;
          const uint32_t slot = wave_reserve(keep, &fill, lane);
          if (keep) cand[slot] = r;
        });
        __syncthreads();
        ncand = (int)kept_total;
      }
    }
  }
  // output: the kept records, in key order
  if (tid == 0) fill = 0;
  __syncthreads();
  auto emit = [&](bool ok, uint64_t r) {
    const bool keep = ok && (r & mask) >= prefix;
    const uint32_t slot = wave_reserve(keep, &fill, lane);
    if (keep) {
      oi[slot] = (int32_t)record_key(r);
      if (os) os[slot] = record_score(r);
    }
  };
  if (ncand < 0) {
    for_row_records(srow, vis, aligned, tid, (int)blockDim.x, emit);
  } else {
    for (int i0 = 0; i0 < ncand; i0 += blockDim.x) {
      const int i = i0 + tid;
      emit(i < ncand, i < ncand ? cand[i] : 0ull);
    }
  }
  for (int j = need + tid; j < topk; j += blockDim.x) {
    oi[j] = -1;
    if (os) os[j] = -INFINITY;
  }
}

hipError_t launch_select_rows(const Problem& p, const float* scores, const uint32_t* row_hist, int topk,
                              int32_t* out_idx, float* out_score, hipStream_t st) {
  const int prof_slot = prof_open("k_select_rows", st);
  hipLaunchKernelGGL(k_select_rows, dim3(p.B * p.Q), dim3(1024), 0, st, scores, row_hist, p.pos, p.N, topk, out_idx,
                     out_score);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

}  // namespace dsa
