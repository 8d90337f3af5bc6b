// prune_prep.hip -- preparation of the certified (DoSA) pruning: seeds, key
// norms and the per-query bound plan.
//
// The bound (DoSA reading notes, annotation LBKERZAW, step 2; 机器之心 DoSA
// article, section 03), for one query row with heads j, weights w_j and the
// shared key k, with d_i = q_i . k:
//   * retained heads R (scored exactly): up to 30 positive-weight heads;
//   * omitted positive-weight heads P: projection onto the retained rows
//     q_j = sum_{i in R} C_ji q_i + r_j with nonnegative C (approximate
//     nonnegative least squares), so with ReLU subadditive and positively
//     homogeneous,
//       w_j ReLU(q_j.k) <= w_j sum_i [C_ji^+ ReLU(d_i) + C_ji^- ReLU(-d_i)]
//                          + w_j |r_j| |k|;
//   * negative-weight heads (none is retained): all of them, N' = N,
//     folded by |w| into one row q_neg; sum |w_j| ReLU(q_j.k) >= ReLU(q_neg . k).
// Summing:  I <= sum_{i in R} [a_i ReLU(d_i) + b_i ReLU(-d_i)] + rho |k|
//                - ReLU(q_neg . k),
// a_i = w_i + sum_P w_j C_ji^+,  b_i = sum_P w_j C_ji^-,  rho = sum_P w_j |r_j|.
// With c_i = (a_i + b_i)/2 and e_i = (a_i - b_i)/2 the retained part is
// sum_i c_i |d_i| + E . k, E = sum_i e_i q_i, so the GPU screen needs one
// fp32 FMA per retained row plus one extra "linear" row E.  With C >= 0,
// b_i = 0 and c_i = e_i = a_i / 2 >= 0, and the fold is tight whenever the
// retained dots share a sign (no cancellation inside a projection).  E and q_neg are
// rounded to the input dtype; their rounding errors (measured here in fp64)
// and a guard for every fp32 rounding of the score and of the bound are
// added to the |k| coefficient, so the computed bound dominates the computed
// score bit for bit (see `guard` below).  Any R, any N' and any C give a
// valid bound; the heuristics below only decide how tight it is.
//
// For fp8 inputs everything is in code units (q8, k8 codes as numbers): the
// score is (q_scale k_scale) * sum_j w_j ReLU(q8_j . k8), and the same
// scaling, monotone in its argument, is applied to the bound.
#include <math.h>

#include "kernels.h"
#include "score_tile.h"

namespace dsa {

// ---------------------------------------------------------------- decoding

// Exact value of an OCP e4m3fn code (bias 7, subnormals m * 2^-9), built
// as fp32 bits: a normal code (e >= 1) is (1 + m/8) 2^(e-7), i.e. exponent
// field e + 120 and mantissa m << 20; a subnormal one is the exact product
// m * 2^-9.  (Codes 0x7F / 0xFF are NaN in e4m3fn and never produced here.)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, mag) | ((c & 0x80u) << 24));
}
__device__ __forceinline__ float bf16_value(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

template <int DT>
__device__ __forceinline__ float elem(const uint8_t* row, int d) {
  if constexpr (DT == kBF16)
    return bf16_value(reinterpret_cast<const uint16_t*>(row)[d]);
  else
    return e4m3_value(row[d]);
}

// ---------------------------------------------------------------- seeds

// One workgroup per sequence.  Default seeds: S_eff = min(S, p0 + 1) keys
// floor(i (p0 + 1) / S_eff), p0 = the last key every row of the sequence sees
// (distinct, ascending, visible to all rows).  Given seeds are checked
// (ascending, distinct, in range); if they fail, the sequence gets no seeds
// and its rows are flagged for recovery.  Also builds the seed bitmap.
__global__ __launch_bounds__(256) void k_seed_prep(const int32_t* __restrict__ pos, int Q, int N, int S,
                                                   const int32_t* __restrict__ user_seeds, int32_t* __restrict__ seeds,
                                                   int32_t* __restrict__ seed_count, uint32_t* __restrict__ bits,
                                                   int words, int32_t* __restrict__ batch_flag) {
  __shared__ int s_min, s_bad;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) {
    s_min = N - 1;
    s_bad = 0;
  }
  __syncthreads();
  int mn = N - 1;
  for (int t = tid; t < Q; t += blockDim.x) mn = min(mn, min(pos[(size_t)b * Q + t], N - 1));
  atomicMin(&s_min, mn);
  uint32_t* bb = bits + (size_t)b * words;
  for (int i = tid; i < words; i += blockDim.x) bb[i] = 0u;
  __syncthreads();
  const int p1 = s_min + 1;  // keys every row sees (may be <= 0)
  int32_t* sb = seeds + (size_t)b * S;
  int cnt;
  if (user_seeds) {
    const int32_t* us = user_seeds + (size_t)b * S;
    for (int i = tid; i < S; i += blockDim.x) {
      const int v = us[i];
      if (v < 0 || v >= N || (i > 0 && us[i - 1] >= v)) atomicOr(&s_bad, 1);
    }
    __syncthreads();
    cnt = s_bad ? 0 : S;
    for (int i = tid; i < cnt; i += blockDim.x) sb[i] = us[i];
  } else {
    cnt = p1 > 0 ? min(S, p1) : 0;
    for (int i = tid; i < cnt; i += blockDim.x) sb[i] = (int32_t)(((int64_t)i * p1) / cnt);
  }
  __syncthreads();
  for (int i = tid; i < cnt; i += blockDim.x) atomicOr(&bb[sb[i] >> 5], 1u << (sb[i] & 31));
  if (tid == 0) {
    seed_count[b] = cnt;
    batch_flag[b] = s_bad;
  }
}

// Anchor seeds (seeds from a few anchor queries): the A anchor rows of a
// sequence are t_i = floor((2i + 1) Q / (2A)), i < A (distinct for A <= Q).
__device__ __forceinline__ int anchor_row(int i, int Q, int A) { return (int)(((int64_t)(2 * i + 1) * Q) / (2 * A)); }

// flag[b * Q + t] = 1 if row t is an anchor row of its sequence, else 0.
// t_i lies within one of t * A / Q, so three candidates decide it.
__global__ __launch_bounds__(256) void k_anchor_rows(int Q, int A, size_t R, int32_t* __restrict__ flag) {
  const size_t row = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= R) return;
  const int t = (int)(row % (size_t)Q);
  const int c = (int)(((int64_t)t * A) / Q);
  int is = 0;
  for (int i = max(0, c - 1); i <= min(A - 1, c + 1); ++i) is |= anchor_row(i, Q, A) == t;
  flag[row] = is;
}

// One workgroup per sequence: the distinct keys of the anchor rows' Top-K
// sets (top_idx rows, -1 padded) as the sequence's seeds, ascending, and
// their bitmap.  The bitmap is set first; then each thread takes a run of
// words, the runs' key counts are prefix-summed over the workgroup, and each
// thread writes its run's keys in order.  At most A * topk <= S keys.
__global__ __launch_bounds__(256) void k_anchor_seeds(int Q, int N, int A, int topk, const int32_t* __restrict__ top_idx,
                                                      int S, int32_t* __restrict__ seeds,
                                                      int32_t* __restrict__ seed_count, uint32_t* __restrict__ bits,
                                                      int words, int32_t* __restrict__ batch_flag) {
  __shared__ int scan[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  uint32_t* bb = bits + (size_t)b * words;
  for (int i = tid; i < words; i += 256) bb[i] = 0u;
  __syncthreads();
  for (int a = 0; a < A; ++a) {
    const int32_t* ti = top_idx + ((size_t)b * Q + anchor_row(a, Q, A)) * (size_t)topk;
    for (int j = tid; j < topk; j += 256) {
      const int key = ti[j];
      if (key >= 0 && key < N) atomicOr(&bb[key >> 5], 1u << (key & 31));
    }
  }
  __syncthreads();
  const int per = (words + 255) / 256;
  const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bb[w]);
  scan[tid] = cnt;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {  // inclusive prefix sum over the workgroup
    const int v = tid >= d ? scan[tid - d] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int o = scan[tid] - cnt;
  int32_t* sb = seeds + (size_t)b * S;
  for (int w = w0; w < w1; ++w) {
    for (uint32_t x = bb[w]; x; x &= x - 1u) {
      if (o < S) sb[o] = w * 32 + __builtin_ctz(x);
      ++o;
    }
  }
  if (tid == 255) {
    seed_count[b] = min(scan[255], S);
    batch_flag[b] = 0;
  }
}

// ---------------------------------------------------------------- key norms

// |k_s| (code units for fp8): each lane squares the values of one 16-byte
// chunk of a key row (exact in fp64), the lanes of a key add their sums, and
// the root is rounded up to fp32 after a margin that covers the fp64
// rounding of the 128-term sum (below 128 * 2^-53 relative).
template <int DT>
__global__ __launch_bounds__(256) void k_key_norms(const uint8_t* __restrict__ k, size_t nkeys,
                                                   float* __restrict__ knorm) {
  constexpr int RB = Frag<DT>::kRowBytes, CPR = RB / 16;  // lanes per key
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t key = t / CPR;
  const int ch = (int)(t % CPR);
  double acc = 0.0;
  if (key < nkeys) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(k + key * RB + ch * 16);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == kBF16) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const double x = bf16_value((uint16_t)(w4[i] >> (16 * h)));
          acc = fma(x, x, acc);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const double x = e4m3_value((w4[i] >> (8 * h)) & 0xFFu);
          acc = fma(x, x, acc);
        }
      }
    }
  }
#pragma unroll
  for (int d = CPR / 2; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);  // the key's lanes (aligned group)
  if (key < nkeys && ch == 0) knorm[key] = __double2float_ru(sqrt(acc * (1.0 + 1e-13)));
}

// ---------------------------------------------------------------- seed pack

// Seed rows packed per sequence: row i of sequence b is key seeds[b][i] for
// i < seed_count[b], else the last seed (key 0 if there is none); these pad
// rows are never visible.  One 16-byte chunk per thread.
template <int DT>
__global__ __launch_bounds__(256) void k_seed_gather(const uint8_t* __restrict__ k, const float* __restrict__ ksc,
                                                     int N, const int32_t* __restrict__ seeds,
                                                     const int32_t* __restrict__ seed_count, int S,
                                                     uint8_t* __restrict__ seed_keys, float* __restrict__ seed_kscale) {
  constexpr int RB = Frag<DT>::kRowBytes, CPR = RB / 16;
  const int b = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // chunk index within the sequence
  if (c >= (int64_t)S * CPR) return;
  const int i = (int)(c / CPR), ch = (int)(c % CPR);
  const int cnt = seed_count[b];
  const int key = cnt > 0 ? seeds[(size_t)b * S + min(i, cnt - 1)] : 0;
  const u32x4* src = reinterpret_cast<const u32x4*>(k + ((size_t)b * N + key) * RB) + ch;
  reinterpret_cast<u32x4*>(seed_keys + ((size_t)b * S + i) * RB)[ch] = *src;
  if (DT == kFP8 && ch == 0) seed_kscale[(size_t)b * S + i] = ksc[(size_t)b * N + key];
}

// seed_pos[row] = (number of the row's sequence's seeds at or below the
// row's position) - 1, by binary search over the ascending seeds.
__global__ __launch_bounds__(256) void k_seed_positions(const int32_t* __restrict__ pos, int Q, size_t rows,
                                                        const int32_t* __restrict__ seeds,
                                                        const int32_t* __restrict__ seed_count, int S,
                                                        int32_t* __restrict__ seed_pos) {
  const size_t row = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  const int b = (int)(row / (size_t)Q);
  const int32_t* sb = seeds + (size_t)b * S;
  const int p = pos[row];
  int lo = 0, hi = seed_count[b];  // first seed > p lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sb[mid] <= p)
      lo = mid + 1;
    else
      hi = mid;
  }
  seed_pos[row] = lo - 1;
}

// ---------------------------------------------------------------- planner

constexpr int kRetained = 30;   // retained heads: plan rows 0..29 (fp8: 0..27)
constexpr int kAuxRow = 30;     // folded negative-head row
constexpr int kLinRow = 31;     // linear row E
constexpr int kLinLoRow = 28;   // fp8: low part of E, a |d| row
constexpr int kAuxLoRow = 29;   // fp8: low part of q_neg, a |d| row
constexpr int kPlanRows = 32;
constexpr int kSweeps = 10;     // coordinate-descent sweeps of the projection
constexpr int kSamples = 128;   // sample keys for the activation statistics
constexpr int kPlanWaves = 4;   // query rows per planner workgroup (one per wave)

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}
// Orders LDS traffic between the lanes of one wave (the planner's waves
// share no LDS, so no workgroup barrier is needed).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}
// gamma_n = n u / (1 - n u), u = 2^-24: relative error bound of n fp32 roundings.
__device__ __forceinline__ float gamma_f(int n) {
  const float u = 5.9604645e-08f;
  return n * u / (1.0f - n * u);
}

// Round fp64 v to a nearby value of the dtype (bf16: via fp32, then RNE;
// e4m3: RNE on the code grid, |v| <= 448 by construction of the row scale).
// The rounding mode does not matter for correctness: the planner measures
// the error of whatever value it stores.  Returns the code bits in *code and
// the value they stand for.
template <int DT>
__device__ __forceinline__ double round_to_dtype(double v, uint32_t* code) {
  if constexpr (DT == kBF16) {
    uint32_t u = __builtin_bit_cast(uint32_t, (float)v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    *code = u >> 16;
    return (double)bf16_value((uint16_t)(u >> 16));
  } else {
    const double a = fmin(fabs(v), 448.0);
    uint32_t c;
    if (a < 0.015625) {  // below 2^-6: subnormal step 2^-9 (m == 8 is the code of 2^-6)
      c = (uint32_t)nearbyint(a * 512.0);
    } else {
      int e = ilogb(a);
      uint32_t m = (uint32_t)nearbyint((ldexp(a, -e) - 1.0) * 8.0);
      if (m == 8) {
        m = 0;
        ++e;
      }
      c = ((uint32_t)(e + 7) << 3) | m;
      if (c > 0x7Eu) c = 0x7Eu;
    }
    if (v < 0 && c) c |= 0x80u;
    *code = c;
    return (double)e4m3_value(c);
  }
}

// Scatter of a 32x32 MFMA result block into a [64][33] staging array: lane l,
// register v holds row 32*blk + 8*(v/4) + 4*(l/32) + v%4, column l%32.
__device__ __forceinline__ void stage_block(float (*red)[33], const f32x16& x, int blk, int lane) {
#pragma unroll
  for (int v = 0; v < 16; ++v) red[32 * blk + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)][lane & 31] = x[v];
}

// One wave per query row, kPlanWaves rows per workgroup.  Writes the 32
// bound rows (dtype), the per-row coefficients (c_0..c_29, aux-row
// multiplier, linear-row multiplier), the |k| coefficient kappa and the aux
// rounding bound e_neg, and the recovery flag (non-finite plan, forced, or
// invalid seeds for the sequence).
//
// Arithmetic: the projection, the residuals and the folded rows are
// computed in fp32; every quantity that enters the bound carries an explicit
// upper bound of its rounding error (gamma_n of the dot products involved),
// so the bound stays certified.
template <int DT>
// Three waves per SIMD (the most its LDS allows): the planner mostly waits on
// loads and LDS round trips, and the extra wave hides more of that than the
// registers it spills cost (0.52 -> 0.37 ms on an 8192-row block).
__global__ __launch_bounds__(kPlanWaves * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_plan(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const float* __restrict__ w,
    const int32_t* __restrict__ pos, int Q, int N, int nret, size_t nrows, const int32_t* __restrict__ seeds,
    const int32_t* __restrict__ seed_count, int seed_stride, const int32_t* __restrict__ batch_flag,
    const uint8_t* __restrict__ force_recover, uint8_t* __restrict__ plan_rows, float* __restrict__ plan_coef,
    float* __restrict__ plan_misc, int32_t* __restrict__ plan_flag) {
  constexpr int RB = Frag<DT>::kRowBytes;
  __shared__ float red_all[kPlanWaves][kHeads][33];  // MFMA staging; later the projection C[j][a]
  __shared__ __align__(16) float G_all[kPlanWaves][kRetained][32];
  __shared__ float inv_all[kPlanWaves][32];
  __shared__ float cch_all[kPlanWaves][32];
  __shared__ float w_all[kPlanWaves][kHeads];
  __shared__ int ridx_all[kPlanWaves][32];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * kPlanWaves + wv;
  if (row >= nrows) return;  // whole wave
  float(*red)[33] = red_all[wv];
  float(*G)[32] = G_all[wv];
  float* inv = inv_all[wv];
  float* cch = cch_all[wv];
  float* ws = w_all[wv];
  int* ridx = ridx_all[wv];

  const int b = (int)(row / (size_t)Q);
  const uint8_t* qrow = q + row * kHeads * RB;
  const int vis = min(max(pos[row] + 1, 0), N);
  const float wj = w[row * kHeads + lane];
  ws[lane] = wj;

  // 1. query fragments; head norms |q_j| from the diagonal of Q Q^T (MFMA;
  //    products of dtype values are exact in fp32, the sum rounds by at
  //    most gamma_128 relative, covered by the margin)
  Frag<DT> qa[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) load_frag<DT>(qa[blk], qrow + (size_t)(32 * blk + (lane & 31)) * RB, lane);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) stage_block(red, mma_block<DT>(qa[blk], qa[blk], zero16()), blk, lane);
  wave_sync();
  const float qnorm = sqrtf(fmaxf(red[lane][lane & 31], 0.0f)) * (1.0f + 1e-5f);
  wave_sync();

  // 2. activation statistics of each head over 128 sample keys (seeds, or
  //    evenly spaced visible keys): X = Q K_s^T by MFMA, 32 samples at a
  //    time (dtype code units for fp8: the scales are positive, so signs and
  //    the head ranking are those of the real values)
  const int nseed = seed_count[b];
  const int32_t* sb = seeds + (size_t)b * seed_stride;
  const int nsamp = min(kSamples, nseed > 0 ? nseed : vis);
  float pa[2][16];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int v = 0; v < 16; ++v) pa[blk][v] = 0.0f;
  for (int s0 = 0; s0 < nsamp; s0 += 32) {
    const int si = s0 + (lane & 31);
    const bool okc = si < nsamp;
    const int key = !okc ? 0 : nseed > 0 ? sb[(int)(((int64_t)si * nseed) / nsamp)] : (int)(((int64_t)si * vis) / nsamp);
    Frag<DT> f;
    load_frag<DT>(f, k + ((size_t)b * N + key) * RB, lane);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const f32x16 x = mma_block<DT>(qa[blk], f, zero16());
#pragma unroll
      for (int v = 0; v < 16; ++v) pa[blk][v] += okc ? relu_bits(x[v]) : 0.0f;
    }
  }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[32 * blk + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)][lane & 31] = pa[blk][v];
  wave_sync();
  float act = 0.0f;
  for (int c = 0; c < 32; ++c) act += red[lane][c];
  wave_sync();

  // 3. retained set: the (at most nret) positive-weight heads with the
  //    largest w_j * activation
  const float key_j = wj > 0.0f ? wj * act : -1.0f;
  int rank = 0;
  for (int i = 0; i < kHeads; ++i) {
    const float ki = __shfl(key_j, i, 64);
    rank += (ki > key_j) || (ki == key_j && i < lane);
  }
  const int npos_heads = __popcll(__ballot(wj > 0.0f));
  nret = min(nret, npos_heads);
  if constexpr (DT == kFP8) nret = min(nret, kLinLoRow);  // rows 28, 29 hold the low parts
  const bool retained = wj > 0.0f && rank < nret;
  if (retained) ridx[rank] = lane;
  wave_sync();

  // 4. dots of every head with every retained row, G_full = Q Q_R^T, by one
  //    MFMA pass (fp32: these only steer the projection, whose residual is
  //    bounded rigorously below).  G = rows ridx of G_full, zero-padded to
  //    30 x 32; head j's right-hand side b_j = row j of G_full.
  {
    Frag<DT> fr;
    const int ri = (lane & 31) < nret ? ridx[lane & 31] : -1;
    if (ri >= 0) {
      load_frag<DT>(fr, qrow + (size_t)ri * RB, lane);
    } else {
#pragma unroll
      for (int i = 0; i < Frag<DT>::kSteps; ++i) fr.v[i] = {};
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) stage_block(red, mma_block<DT>(qa[blk], fr, zero16()), blk, lane);
  }
  wave_sync();
  for (int e = lane; e < kRetained * 32; e += 64) {
    const int a = e >> 5, c = e & 31;
    G[a][c] = (a < nret && c < nret) ? red[ridx[a]][c] : 0.0f;
  }
  if (lane < 32) inv[lane] = 0.0f;
  wave_sync();
  if (lane < nret) inv[lane] = G[lane][lane] > 0.0f ? 1.0f / G[lane][lane] : 0.0f;
  // 5. each omitted positive head (lane) projects onto the retained rows
  //    with nonnegative coefficients: coordinate descent on
  //    min |q_j - C Q_R|^2, C >= 0, from C = 0, a fixed number of sweeps.
  //    Any C >= 0 gives a valid bound (convergence only tightens it).
  const bool in_P = !retained && wj > 0.0f;
  float C[kRetained], bq[kRetained];
#pragma unroll
  for (int a = 0; a < kRetained; ++a) {
    C[a] = 0.0f;
    bq[a] = (in_P && a < nret) ? red[lane][a] : 0.0f;
  }
  wave_sync();
  if (__ballot(in_P) != 0 && nret > 0) {
    for (int sw = 0; sw < kSweeps; ++sw) {
      // re-read G from LDS each sweep (keeps its 960 entries out of registers)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < kRetained; ++i) {
        if (i < nret) {
          const float4* gi = reinterpret_cast<const float4*>(G[i]);
          float g[4] = {-bq[i], 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int m4 = 0; m4 < 8; ++m4) {
            const float4 x = gi[m4];
            if (4 * m4 + 0 < kRetained) g[0] = __builtin_fmaf(C[4 * m4 + 0], x.x, g[0]);
            if (4 * m4 + 1 < kRetained) g[1] = __builtin_fmaf(C[4 * m4 + 1], x.y, g[1]);
            if (4 * m4 + 2 < kRetained) g[2] = __builtin_fmaf(C[4 * m4 + 2], x.z, g[2]);
            if (4 * m4 + 3 < kRetained) g[3] = __builtin_fmaf(C[4 * m4 + 3], x.w, g[3]);
          }
          C[i] = fmaxf(0.0f, C[i] - ((g[0] + g[1]) + (g[2] + g[3])) * inv[i]);
        }
      }
    }
  }
  // the projection as an LDS matrix C[j][a] (zero rows outside P)
#pragma unroll
  for (int a = 0; a < kRetained; ++a) red[lane][a] = in_P ? C[a] : 0.0f;
  wave_sync();

  // 6. folded coefficients (lanes = retained rows): a_i = w_i + sum_P w_j
  //    C_ji, all terms >= 0, so the fp32 sum is low by at most gamma_65
  //    relative; c_i = e_i = a_i / 2 rounded up (a larger c_i keeps the
  //    bound valid: sum 2 c_i ReLU(d_i) >= sum a_i ReLU(d_i))
  if (lane < 32) {
    float ai = 0.0f;
    if (lane < nret) {
      ai = ws[ridx[lane]];
      for (int j = 0; j < kHeads; ++j) ai = __builtin_fmaf(fmaxf(ws[j], 0.0f), red[j][lane], ai);
      ai = 0.5f * ai * (1.0f + 2e-5f);
    }
    cch[lane] = ai;
  }
  wave_sync();

  // 7. lanes = dims d0 = lane, d1 = lane + 64: the retained rows' values,
  //    then per omitted head the residual r_j = q_j - sum_a C_ja q_a.  Its
  //    fp32 evaluation (an fma chain from q_j) is off by at most gamma_31
  //    (|q_j| + sum_a C_ja |q_a|) per component, so
  //    |r_j| <= |r_computed| + gamma_31 |m_j| (m_j: that sum).
  const int d0 = lane, d1 = lane + 64;
  float qr0[kRetained], qr1[kRetained];
#pragma unroll
  for (int a = 0; a < kRetained; ++a) {
    const bool ok = a < nret;
    const uint8_t* ra = qrow + (size_t)(ok ? ridx[a] : 0) * RB;
    qr0[a] = ok ? elem<DT>(ra, d0) : 0.0f;
    qr1[a] = ok ? elem<DT>(ra, d1) : 0.0f;
  }
  float rho = 0.0f;
  uint64_t pmask = __ballot(in_P);
  while (pmask) {
    const int j = __builtin_ctzll(pmask);
    pmask &= pmask - 1;
    const float* cj = red[j];
    const float qj0 = elem<DT>(qrow + (size_t)j * RB, d0), qj1 = elem<DT>(qrow + (size_t)j * RB, d1);
    float r0 = qj0, r1 = qj1, m0 = fabsf(qj0), m1 = fabsf(qj1);
#pragma unroll
    for (int a = 0; a < kRetained; ++a) {
      const float c = cj[a];
      r0 = __builtin_fmaf(-c, qr0[a], r0);
      r1 = __builtin_fmaf(-c, qr1[a], r1);
      m0 = __builtin_fmaf(c, fabsf(qr0[a]), m0);
      m1 = __builtin_fmaf(c, fabsf(qr1[a]), m1);
    }
    const float sr = wave_sum_f(__builtin_fmaf(r0, r0, r1 * r1));
    const float sm = wave_sum_f(__builtin_fmaf(m0, m0, m1 * m1));
    const float rn = (sqrtf(sr) + gamma_f(32) * sqrtf(sm)) * (1.0f + 2e-5f);
    rho = __builtin_fmaf(__shfl(wj, j, 64), rn, rho);
  }
  rho *= 1.0f + 1e-5f;  // nonnegative terms: sum low by at most gamma_34

  // 8. folded negative row: every negative-weight head (none is retained).
  //    Any subset gives a valid penalty: leaving a head out raises the fold
  //    on keys where that head is inactive and lowers it where it is
  //    active.  On keys that score near the K-th score the full fold
  //    excludes the most (almost as many as exact per-head penalties would).
  const bool in_N = !retained && wj < 0.0f;

  // 9. E = sum_a c_a q_a and q_neg = sum_N' |w_j| q_j in fp32 (lanes =
  //    dims) with their component error bounds gamma_n * (sum of |terms|)
  float E0 = 0.0f, E1 = 0.0f, mE0 = 0.0f, mE1 = 0.0f;
#pragma unroll
  for (int a = 0; a < kRetained; ++a) {
    const float c = cch[a];
    E0 = __builtin_fmaf(c, qr0[a], E0);
    E1 = __builtin_fmaf(c, qr1[a], E1);
    mE0 = __builtin_fmaf(c, fabsf(qr0[a]), mE0);
    mE1 = __builtin_fmaf(c, fabsf(qr1[a]), mE1);
  }
  float N0 = 0.0f, N1 = 0.0f, mN0 = 0.0f, mN1 = 0.0f;
  uint64_t nmask = __ballot(in_N);
  while (nmask) {
    const int j = __builtin_ctzll(nmask);
    nmask &= nmask - 1;
    const float aw = fabsf(ws[j]);
    const float qj0 = elem<DT>(qrow + (size_t)j * RB, d0), qj1 = elem<DT>(qrow + (size_t)j * RB, d1);
    N0 = __builtin_fmaf(aw, qj0, N0);
    N1 = __builtin_fmaf(aw, qj1, N1);
    mN0 = __builtin_fmaf(aw, fabsf(qj0), mN0);
    mN1 = __builtin_fmaf(aw, fabsf(qj1), mN1);
  }
  // Stored rows.  bf16: E and q_neg rounded to bf16.  fp8 (3 mantissa
  // bits): each is split into a high part x_h = e4m3(x / m_h) m_h (the
  // linear / aux row) and a low part x_l = e4m3((x - x_h) / m_l) m_l (plan
  // row 28 for E, 29 for q_neg), m_h, m_l powers of two that bring the
  // part's largest magnitude within the e4m3 range.  The low parts enter
  // the bound as |d| rows with coefficient m_l:
  //   E.k <= x_h.k + |x_l.k| + |E - x_h - x_l| |k|, and
  //   ReLU(q_neg.k) >= ReLU(x_h.k - e_neg |k|) - |x_l.k|
  // (ReLU is monotone and 1-Lipschitz), so both stay upper bounds while the
  // |k| coefficients shrink to the rounding error of the two-part sum.
  // |x - stored| <= |x_fp32 - stored| + gamma_30 |mE| (q_neg: gamma_64),
  // differences and norms in fp64.
  auto pow2_step = [](float am) {  // smallest power of two m with am / m <= 448
    return am > 0.0f ? ldexp(1.0, (int)ceil(log2((double)am / 448.0))) : 1.0;
  };
  auto wave_max_f = [](float x) {
#pragma unroll
    for (int dd = 32; dd >= 1; dd >>= 1) x = fmaxf(x, __shfl_xor(x, dd, 64));
    return x;
  };
  uint8_t* prow = plan_rows + row * kPlanRows * RB;
  double err2[2] = {0.0, 0.0}, nrm2[2] = {0.0, 0.0}, mag2[2] = {0.0, 0.0}, lo2[2] = {0.0, 0.0};
  double mult[2] = {1.0, 1.0}, mult_lo[2] = {1.0, 1.0};
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const float xs[2] = {v == 0 ? E0 : N0, v == 0 ? E1 : N1};
    const float gs[2] = {v == 0 ? mE0 : mN0, v == 0 ? mE1 : mN1};
    if constexpr (DT == kFP8) mult[v] = pow2_step(wave_max_f(fmaxf(fabsf(xs[0]), fabsf(xs[1]))));
    uint8_t* dst = prow + (size_t)(v == 0 ? kLinRow : kAuxRow) * RB;
    double stored[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t code;
      stored[h] = round_to_dtype<DT>((double)xs[h] / mult[v], &code) * mult[v];
      if constexpr (DT == kBF16)
        reinterpret_cast<uint16_t*>(dst)[h ? d1 : d0] = (uint16_t)code;
      else
        dst[h ? d1 : d0] = (uint8_t)code;
      nrm2[v] = fma(stored[h], stored[h], nrm2[v]);
    }
    if constexpr (DT == kFP8) {
      const double r[2] = {(double)xs[0] - stored[0], (double)xs[1] - stored[1]};  // exact
      mult_lo[v] = pow2_step(wave_max_f(fmaxf((float)fabs(r[0]), (float)fabs(r[1]))));
      uint8_t* dlo = prow + (size_t)(v == 0 ? kLinLoRow : kAuxLoRow) * RB;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t code;
        const double lo = round_to_dtype<DT>(r[h] / mult_lo[v], &code) * mult_lo[v];
        dlo[h ? d1 : d0] = (uint8_t)code;
        stored[h] += lo;
        lo2[v] = fma(lo, lo, lo2[v]);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const double e = (double)xs[h] - stored[h];
      err2[v] = fma(e, e, err2[v]);
      mag2[v] = fma((double)gs[h], (double)gs[h], mag2[v]);
    }
    err2[v] = wave_sum_d(err2[v]);
    nrm2[v] = wave_sum_d(nrm2[v]);
    mag2[v] = wave_sum_d(mag2[v]);
    lo2[v] = wave_sum_d(lo2[v]);
  }
  const double e_lin = (sqrt(err2[0]) + (double)gamma_f(32) * sqrt(mag2[0]) * (1.0 + 1e-6)) * (1.0 + 1e-12);
  const double e_neg = (sqrt(err2[1]) + (double)gamma_f(66) * sqrt(mag2[1]) * (1.0 + 1e-6)) * (1.0 + 1e-12);
  // norms of the high rows and (fp8) of the low rows, for the guard
  const double n_lin = sqrt(nrm2[0]), n_neg = sqrt(nrm2[1]), n_lo = sqrt(lo2[0]) + sqrt(lo2[1]);

  // retained rows: the query's own codes (fp8: rows 28, 29 hold the low parts)
  for (int a = 0; a < (DT == kFP8 ? kLinLoRow : kRetained); ++a) {
    uint8_t* dst = prow + (size_t)a * RB;
    const uint8_t* src = qrow + (size_t)(a < nret ? ridx[a] : 0) * RB;
    for (int x = lane; x < RB / 4; x += 64)
      reinterpret_cast<uint32_t*>(dst)[x] = a < nret ? reinterpret_cast<const uint32_t*>(src)[x] : 0u;
  }

  // 10. guard: the GPU's fp32 score differs from the exact one by at most
  //    (g_128 + 2 g_64) W1 |k| (128-term dots, 64-term head sum, final
  //    combine), and the fp32 bound from its exact value by at most
  //    (g_128 + g_24) Wb |k| + g_24 (e_neg + rho + e_lin) |k|, where
  //    g_n = n u / (1 - n u), u = 2^-24 (the screen adds each lane's rows
  //    in two chains of eight, then the chain sum, the other half's sum and
  //    the aux, linear and |k| terms: at most 14 roundings per term, within
  //    g_24).  Doubled for margin.
  const double u = 5.9604644775390625e-08;
  auto gam = [u](double n) { return n * u / (1.0 - n * u); };
  const double W1 = wave_sum_d(fabs((double)wj) * (double)qnorm);
  double Wb = n_lin + n_neg + n_lo;
  for (int a = 0; a < nret; ++a) Wb += (double)cch[a] * (double)__shfl(qnorm, ridx[a], 64);
  const double guard =
      2.0 * ((gam(128) + 2.0 * gam(64) + gam(4)) * W1 + (gam(128) + gam(24)) * Wb + gam(24) * (e_neg + rho + e_lin));
  const double kappa = ((double)rho + e_lin + guard) * (1.0 + 1e-9);

  bool finite = isfinite(kappa) && isfinite(e_neg) && isfinite(mult[0]) && isfinite(mult[1]) &&
                isfinite(mult_lo[0]) && isfinite(mult_lo[1]);
  for (int a = 0; a < kRetained; ++a) finite = finite && isfinite(cch[a]);
  if (lane == 0) {
    float* co = plan_coef + row * kPlanRows;
    for (int a = 0; a < kRetained; ++a) co[a] = cch[a];
    if constexpr (DT == kFP8) {
      co[kLinLoRow] = (float)mult_lo[0];
      co[kAuxLoRow] = (float)mult_lo[1];
    }
    co[kAuxRow] = (float)mult[1];
    co[kLinRow] = (float)mult[0];
    float* mi = plan_misc + row * 4;
    mi[0] = __double2float_ru(kappa);
    mi[1] = __double2float_ru(e_neg);
    mi[2] = 0.0f;
    mi[3] = 0.0f;
    const bool forced = force_recover && force_recover[row];
    plan_flag[row] = (!finite || forced || batch_flag[b]) ? 1 : 0;
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_seed_prep(const Problem& p, int S, const int32_t* user_seeds, int32_t* seeds, int32_t* seed_count,
                            uint32_t* bits, int32_t* batch_flag, hipStream_t st) {
  const int prof_slot = prof_open("k_seed_prep", st);
  const int words = (p.N + 31) / 32;
  hipLaunchKernelGGL(k_seed_prep, dim3(p.B), dim3(256), 0, st, p.pos, p.Q, p.N, S, user_seeds, seeds, seed_count,
                     bits, words, batch_flag);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

hipError_t launch_anchor_rows(const Problem& p, int A, int32_t* flag, hipStream_t st) {
  const size_t rows = (size_t)p.B * p.Q;
  hipLaunchKernelGGL(k_anchor_rows, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, p.Q, A, rows, flag);
  return hipGetLastError();
}

hipError_t launch_anchor_seeds(const Problem& p, int A, int topk, const int32_t* top_idx, int S, int32_t* seeds,
                               int32_t* seed_count, uint32_t* bits, int32_t* batch_flag, hipStream_t st) {
  const int prof_slot = prof_open("k_anchor_seeds", st);
  const int words = (p.N + 31) / 32;
  hipLaunchKernelGGL(k_anchor_seeds, dim3(p.B), dim3(256), 0, st, p.Q, p.N, A, topk, top_idx, S, seeds, seed_count,
                     bits, words, batch_flag);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

hipError_t launch_key_norms(const Problem& p, float* knorm, hipStream_t st) {
  const int prof_slot = prof_open("k_key_norms", st);
  const size_t n = (size_t)p.B * p.N;
  const int cpr = (p.dtype == kBF16 ? Frag<kBF16>::kRowBytes : Frag<kFP8>::kRowBytes) / 16;
  const dim3 grid((unsigned)((n * cpr + 255) / 256));
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_key_norms<kBF16>, grid, dim3(256), 0, st, p.k, n, knorm);
  else
    hipLaunchKernelGGL(k_key_norms<kFP8>, grid, dim3(256), 0, st, p.k, n, knorm);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

hipError_t launch_seed_pack(const Problem& p, const int32_t* seeds, const int32_t* seed_count, int seed_stride,
                            uint8_t* seed_keys, float* seed_kscale, int32_t* seed_pos, hipStream_t st) {
  const int prof_slot = prof_open("k_seed_pack", st);
  const int cpr = (p.dtype == kBF16 ? Frag<kBF16>::kRowBytes : Frag<kFP8>::kRowBytes) / 16;
  const dim3 grid((unsigned)(((int64_t)seed_stride * cpr + 255) / 256), p.B);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_seed_gather<kBF16>, grid, dim3(256), 0, st, p.k, p.k_scale, p.N, seeds, seed_count,
                       seed_stride, seed_keys, seed_kscale);
  else
    hipLaunchKernelGGL(k_seed_gather<kFP8>, grid, dim3(256), 0, st, p.k, p.k_scale, p.N, seeds, seed_count,
                       seed_stride, seed_keys, seed_kscale);
  const size_t rows = (size_t)p.B * p.Q;
  hipLaunchKernelGGL(k_seed_positions, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, p.pos, p.Q, rows, seeds,
                     seed_count, seed_stride, seed_pos);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

hipError_t launch_plan(const Problem& p, int nret, const int32_t* seeds, const int32_t* seed_count, int seed_stride,
                       const int32_t* batch_flag, const uint8_t* force_recover, uint8_t* plan_rows, float* plan_coef,
                       float* plan_misc, int32_t* plan_flag, hipStream_t st) {
  const int prof_slot = prof_open("k_plan", st);
  const size_t nrows = (size_t)p.B * p.Q;
  const dim3 grid((unsigned)((nrows + kPlanWaves - 1) / kPlanWaves));
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_plan<kBF16>, grid, dim3(kPlanWaves * 64), 0, st, p.q, p.k, p.w, p.pos, p.Q, p.N, nret, nrows,
                       seeds, seed_count, seed_stride, batch_flag, force_recover, plan_rows, plan_coef, plan_misc,
                       plan_flag);
  else
    hipLaunchKernelGGL(k_plan<kFP8>, grid, dim3(kPlanWaves * 64), 0, st, p.q, p.k, p.w, p.pos, p.Q, p.N, nret, nrows,
                       seeds, seed_count, seed_stride, batch_flag, force_recover, plan_rows, plan_coef, plan_misc,
                       plan_flag);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

}  // namespace dsa
