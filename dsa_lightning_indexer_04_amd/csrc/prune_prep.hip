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
//   * negative-weight heads (none is retained): the selected subset N'
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

// Exact value of an OCP e4m3fn code (bias 7, subnormals m * 2^-9).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? ldexpf((float)(8u + m), (int)e - 10) : ldexpf((float)m, -9);
  return (c & 0x80u) ? -mag : mag;
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

// ---------------------------------------------------------------- key norms

// |k_s| (code units for fp8), accumulated in fp64 and rounded up to fp32.
template <int DT>
__global__ __launch_bounds__(256) void k_key_norms(const uint8_t* __restrict__ k, size_t nkeys,
                                                   float* __restrict__ knorm) {
  const size_t s = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nkeys) return;
  const uint8_t* row = k + s * Frag<DT>::kRowBytes;
  double acc = 0.0;
  for (int d = 0; d < kDim; ++d) {
    const double v = elem<DT>(row, d);
    acc = fma(v, v, acc);
  }
  knorm[s] = __double2float_ru(sqrt(acc) * (1.0 + 1e-15));
}

// ---------------------------------------------------------------- planner

constexpr int kRetained = 30;   // retained heads: plan rows 0..29
constexpr int kAuxRow = 30;     // folded negative-head row
constexpr int kLinRow = 31;     // linear row E
constexpr int kPlanRows = 32;
constexpr int kSweeps = 20;     // coordinate-descent sweeps of the projection
constexpr int kSamples = 128;   // sample keys for the activation statistics
constexpr int kQPad = kDim + 1; // padded LDS row (conflict-free column reads)

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
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

// One wave per query row.  Writes the 32 bound rows (dtype), the per-row
// coefficients (c_0..c_29, aux-row multiplier, linear-row multiplier), the
// |k| coefficient kappa and the aux rounding bound e_neg, and the recovery
// flag (non-finite plan, forced, or invalid seeds for the sequence).
template <int DT>
__global__ __launch_bounds__(64) void k_plan(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                                             const float* __restrict__ w, const int32_t* __restrict__ pos, int Q,
                                             int N, int nret, const int32_t* __restrict__ seeds,
                                             const int32_t* __restrict__ seed_count, int seed_stride,
                                             const int32_t* __restrict__ batch_flag,
                                             const uint8_t* __restrict__ force_recover,
                                             uint8_t* __restrict__ plan_rows, float* __restrict__ plan_coef,
                                             float* __restrict__ plan_misc, int32_t* __restrict__ plan_flag) {
  constexpr int RB = Frag<DT>::kRowBytes;
  __shared__ float qs[kHeads][kQPad];
  __shared__ float red[kHeads][33];   // per-head staging of MFMA results
  __shared__ float G[kRetained][kRetained];
  __shared__ double cch[kRetained];  // c_i = e_i (folded retained coefficients)
  __shared__ int ridx[kRetained];
  __shared__ double vec[2][kDim];  // E, q_neg (fp64)
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;
  const int b = (int)(row / (size_t)Q);
  const uint8_t* qrow = q + row * kHeads * RB;
  const int vis = min(max(pos[row] + 1, 0), N);

  // 1. query rows into LDS (fp32 values: exact for bf16 and e4m3 codes)
  for (int j = 0; j < kHeads; ++j)
    for (int d = lane; d < kDim; d += 64) qs[j][d] = elem<DT>(qrow + (size_t)j * RB, d);
  const double wj = w[row * kHeads + lane];
  __syncthreads();
  double qn2 = 0.0;
  for (int d = 0; d < kDim; ++d) qn2 = fma((double)qs[lane][d], (double)qs[lane][d], qn2);
  const double qnorm = sqrt(qn2);

  // 2. activation statistics of each head over 128 sample keys (seeds, or
  //    evenly spaced visible keys): X = Q K_s^T by MFMA, 32 samples at a
  //    time (dtype code units for fp8: the scales are positive, so signs and
  //    the head ranking are those of the real values).  Lane l holds sample
  //    l % 32 for heads 32*blk + 8*(v/4) + 4*(l/32) + v%4; the per-head sums
  //    over the 32 sample columns go through LDS.
  const int nseed = seed_count[b];
  const int32_t* sb = seeds + (size_t)b * seed_stride;
  const int nsamp = min(kSamples, nseed > 0 ? nseed : vis);
  Frag<DT> qa[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) load_frag<DT>(qa[blk], qrow + (size_t)(32 * blk + (lane & 31)) * RB, lane);
  float pa[2][16], pn[2][16];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int v = 0; v < 16; ++v) pa[blk][v] = pn[blk][v] = 0.0f;
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
      for (int v = 0; v < 16; ++v) {
        pa[blk][v] += okc ? relu_bits(x[v]) : 0.0f;
        pn[blk][v] += (okc && x[v] > 0.0f) ? 1.0f : 0.0f;
      }
    }
  }
  float act = 0.0f;
  int npos = 0;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        red[32 * blk + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)][lane & 31] = pass ? pn[blk][v] : pa[blk][v];
    __syncthreads();
    float sum = 0.0f;
    for (int c = 0; c < 32; ++c) sum += red[lane][c];
    if (pass)
      npos = (int)sum;
    else
      act = sum;
    __syncthreads();
  }

  // 3. retained set: the (at most nret) positive-weight heads with the
  //    largest w_j * activation
  const float key_j = wj > 0.0 ? (float)wj * act : -1.0f;
  int rank = 0;
  for (int i = 0; i < kHeads; ++i) {
    const float ki = __shfl(key_j, i, 64);
    rank += (ki > key_j) || (ki == key_j && i < lane);
  }
  const int npos_heads = __popcll(__ballot(wj > 0.0));
  nret = min(nret, npos_heads);
  const bool retained = wj > 0.0 && rank < nret;
  if (retained) ridx[rank] = lane;
  __syncthreads();

  // 4. dots of every head with every retained row, G_full = Q Q_R^T, by one
  //    MFMA pass (fp32: these only steer the projection, whose residual is
  //    measured exactly below).  G = rows ridx of G_full; head j's
  //    right-hand side b_j = row j of G_full.
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
    for (int blk = 0; blk < 2; ++blk) {
      const f32x16 x = mma_block<DT>(qa[blk], fr, zero16());
#pragma unroll
      for (int v = 0; v < 16; ++v) red[32 * blk + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)][lane & 31] = x[v];
    }
  }
  __syncthreads();
  for (int e = lane; e < nret * nret; e += 64) {
    const int a = e / nret, c = e % nret;
    G[a][c] = red[ridx[a]][c];
  }
  __syncthreads();

  // 5. each omitted positive head (lane) projects onto the retained rows
  //    with nonnegative coefficients: coordinate descent on
  //    min |q_j - C Q_R|^2, C >= 0, from C = 0, a fixed number of sweeps.
  //    Any C >= 0 gives a valid bound (convergence only tightens it); the
  //    residual is then measured in fp64 from the C actually used.
  const bool in_P = !retained && wj > 0.0;
  float C[kRetained];
  float bq[kRetained];
  double rnorm = 0.0;
#pragma unroll
  for (int a = 0; a < kRetained; ++a) {
    C[a] = 0.0f;
    bq[a] = 0.0f;
  }
  if (in_P && nret > 0) {
#pragma unroll
    for (int a = 0; a < kRetained; ++a)
      if (a < nret) bq[a] = red[lane][a];
    for (int sw = 0; sw < kSweeps; ++sw) {
      // re-read G from LDS each sweep (keeps its 900 entries out of registers)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < kRetained; ++i) {
        if (i < nret && G[i][i] > 0.0f) {
          float g = -bq[i];
#pragma unroll
          for (int m = 0; m < kRetained; ++m)
            if (m < nret) g = fmaf(C[m], G[i][m], g);  // G is symmetric: row i
          C[i] = fmaxf(0.0f, C[i] - g / G[i][i]);
        }
      }
    }
  }
  if (in_P) {
    double r2 = 0.0, rmag = 0.0;
    for (int d = 0; d < kDim; ++d) {
      double r = qs[lane][d];
      double m = fabs(r);
#pragma unroll
      for (int a = 0; a < kRetained; ++a) {
        if (a < nret) {
          r = fma(-(double)C[a], (double)qs[ridx[a]][d], r);
          m += fabs((double)C[a] * qs[ridx[a]][d]);
        }
      }
      r2 = fma(r, r, r2);
      rmag = fmax(rmag, m);
    }
    // fp64 rounding of the residual: at most ~(nret+2) ulps of the term sizes
    rnorm = sqrt(r2) + 32.0 * (nret + 2) * 1.1102230246251565e-16 * rmag * sqrt((double)kDim);
  }

  // 6. folded coefficients (C >= 0, so b_i = 0): a_i = w_i + sum_P w_j C_ji,
  //    c_i = e_i = a_i / 2 (wave-uniform, kept in LDS); rho = sum_P w_j |r_j|
  const double rho = wave_sum_d(in_P ? wj * rnorm : 0.0);
#pragma unroll
  for (int a = 0; a < kRetained; ++a) {
    if (a < nret) {
      const double ap = wave_sum_d(in_P ? wj * (double)C[a] : 0.0);
      const double wa = __shfl(wj, ridx[a], 64);
      if (lane == 0) cch[a] = 0.5 * (wa + ap);
    } else if (lane == 0) {
      cch[a] = 0.0;
    }
  }
  __syncthreads();

  // 7. folded negative row: negative heads active on >= half the samples
  //    (all negative heads if none is)
  const bool negom = !retained && wj < 0.0;
  const bool act_half = negom && 2 * npos >= nsamp && nsamp > 0;
  const bool use_half = __ballot(act_half) != 0;
  const bool in_N = use_half ? act_half : negom;

  // 8. E and q_neg in fp64 (lanes over dims), rounded to the dtype
  for (int d = lane; d < kDim; d += 64) {
    double e = 0.0;
#pragma unroll
    for (int a = 0; a < kRetained; ++a)
      if (a < nret) e = fma(cch[a], (double)qs[ridx[a]][d], e);
    vec[0][d] = e;
    double n = 0.0;
    for (int j = 0; j < kHeads; ++j) {
      const double wjj = __shfl(wj, j, 64);
      const bool inj = __shfl((int)in_N, j, 64) != 0;
      if (inj) n = fma(fabs(wjj), (double)qs[j][d], n);
    }
    vec[1][d] = n;
  }
  __syncthreads();
  // row multipliers: 1 for bf16; for fp8 a power of two that brings the
  // row's largest magnitude within the e4m3 range
  double mult[2] = {1.0, 1.0};
  if constexpr (DT == kFP8) {
    for (int v = 0; v < 2; ++v) {
      double amax = 0.0;
      for (int d = lane; d < kDim; d += 64) amax = fmax(amax, fabs(vec[v][d]));
#pragma unroll
      for (int dd = 32; dd >= 1; dd >>= 1) amax = fmax(amax, __shfl_xor(amax, dd, 64));
      mult[v] = amax > 0 ? ldexp(1.0, (int)ceil(log2(amax / 448.0))) : 1.0;
    }
  }
  double err2[2] = {0.0, 0.0}, nrm2[2] = {0.0, 0.0};
  uint8_t* prow = plan_rows + row * kPlanRows * RB;
  for (int v = 0; v < 2; ++v) {
    uint8_t* dst = prow + (size_t)(v == 0 ? kLinRow : kAuxRow) * RB;
    for (int d = lane; d < kDim; d += 64) {
      uint32_t code;
      const double rv = round_to_dtype<DT>(vec[v][d] / mult[v], &code) * mult[v];
      if constexpr (DT == kBF16)
        reinterpret_cast<uint16_t*>(dst)[d] = (uint16_t)code;
      else
        dst[d] = (uint8_t)code;
      err2[v] = fma(vec[v][d] - rv, vec[v][d] - rv, err2[v]);
      nrm2[v] = fma(rv, rv, nrm2[v]);
    }
    err2[v] = wave_sum_d(err2[v]);
    nrm2[v] = wave_sum_d(nrm2[v]);
  }
  const double e_lin = sqrt(err2[0]) * (1.0 + 1e-12), e_neg = sqrt(err2[1]) * (1.0 + 1e-12);
  const double n_lin = sqrt(nrm2[0]), n_neg = sqrt(nrm2[1]);

  // retained rows: the query's own codes
  for (int a = 0; a < kRetained; ++a) {
    uint8_t* dst = prow + (size_t)a * RB;
    const uint8_t* src = qrow + (size_t)(a < nret ? ridx[a] : 0) * RB;
    for (int x = lane; x < RB / 4; x += 64)
      reinterpret_cast<uint32_t*>(dst)[x] = a < nret ? reinterpret_cast<const uint32_t*>(src)[x] : 0u;
  }

  // 9. guard: the GPU's fp32 score differs from the exact one by at most
  //    (g_128 + 2 g_64) W1 |k| (128-term dots, 64-term head sum, final
  //    combine), and the fp32 bound from its exact value by at most
  //    (g_128 + g_24) Wb |k| + g_24 (e_neg + rho + e_lin) |k|, where
  //    g_n = n u / (1 - n u), u = 2^-24 (the screen adds each lane's 16
  //    rows in one chain, then the other half's sum and the |k| term: at
  //    most 20 roundings per term, within g_24).  Doubled for margin.
  const double u = 5.9604644775390625e-08;
  auto gam = [u](double n) { return n * u / (1.0 - n * u); };
  const double W1 = wave_sum_d(fabs(wj) * qnorm);
  double Wb = n_lin + n_neg;
#pragma unroll
  for (int a = 0; a < kRetained; ++a)
    if (a < nret) Wb += fabs(cch[a]) * __shfl(qnorm, ridx[a], 64);
  const double guard =
      2.0 * ((gam(128) + 2.0 * gam(64) + gam(4)) * W1 + (gam(128) + gam(24)) * Wb + gam(24) * (e_neg + rho + e_lin));
  const double kappa = (rho + e_lin + guard) * (1.0 + 1e-9);

  bool finite = isfinite(kappa) && isfinite(e_neg) && isfinite(mult[0]) && isfinite(mult[1]);
  for (int a = 0; a < kRetained; ++a) finite = finite && isfinite(cch[a]);
  if (lane == 0) {
    float* co = plan_coef + row * kPlanRows;
    for (int a = 0; a < kRetained; ++a) co[a] = __double2float_ru(cch[a]);
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

hipError_t launch_key_norms(const Problem& p, float* knorm, hipStream_t st) {
  const int prof_slot = prof_open("k_key_norms", st);
  const size_t n = (size_t)p.B * p.N;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_key_norms<kBF16>, grid, dim3(256), 0, st, p.k, n, knorm);
  else
    hipLaunchKernelGGL(k_key_norms<kFP8>, grid, dim3(256), 0, st, p.k, n, knorm);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

hipError_t launch_plan(const Problem& p, int nret, const int32_t* seeds, const int32_t* seed_count, int seed_stride,
                       const int32_t* batch_flag, const uint8_t* force_recover, uint8_t* plan_rows, float* plan_coef,
                       float* plan_misc, int32_t* plan_flag, hipStream_t st) {
  const int prof_slot = prof_open("k_plan", st);
  const dim3 grid((unsigned)((size_t)p.B * p.Q));
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(k_plan<kBF16>, grid, dim3(64), 0, st, p.q, p.k, p.w, p.pos, p.Q, p.N, nret, seeds,
                       seed_count, seed_stride, batch_flag, force_recover, plan_rows, plan_coef, plan_misc, plan_flag);
  else
    hipLaunchKernelGGL(k_plan<kFP8>, grid, dim3(64), 0, st, p.q, p.k, p.w, p.pos, p.Q, p.N, nret, seeds, seed_count,
                       seed_stride, batch_flag, force_recover, plan_rows, plan_coef, plan_misc, plan_flag);
  prof_close(prof_slot, st);
  return hipGetLastError();
}

}  // namespace dsa
