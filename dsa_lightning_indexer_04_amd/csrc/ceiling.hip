// ceiling.hip -- the sustained rate of the score step on this part (a
// benchmark aid, not part of any Top-K path).
//
// The nominal dense MFMA peak assumes the top clock.  Under a full MFMA load
// the part lowers its clock to stay in its power budget, and how far depends
// on the operands' bit activity and on the vector work issued beside the
// MFMAs.  This kernel measures the rate the score step can sustain with no
// memory traffic at all: every wave holds one synthetic query (64 heads x 128
// dims, full-entropy bf16 or e4m3 codes, signed fp32 head weights) and
// streams 32-key blocks from a 64-key LDS tile in the streaming kernel's
// padded layout, through the same routines the streaming Top-K uses
// (pipelined_partial, combine_single).  Two workgroups of four waves per
// compute unit, two waves per SIMD, as there.
//   mode 0: the MFMAs and key-fragment reloads alone (accumulators chained);
//   mode 1: mode 0 plus the ReLU-weighted head sum and the cross-half
//           combine of every block, i.e. the streaming kernel's block step
//           without candidate appends, tile loads or barriers;
//   mode 2 (bf16): the step in the form w ReLU(x) = (w/2)(x + |x|): one FMA
//           with an absolute-value source per head and key, plus the linear
//           term u . k (u = sum_j (w_j/2) q_j as high and low bf16 rows) on
//           a 16-row block, 8 more 16x16x32 MFMAs per 32 keys, its key
//           fragments read from the same tile and its sums moved to the
//           score's lanes by two LDS permutes.
// Work per launch: workgroups x 4 waves x iters blocks x 2*64*32*128 FLOP.
#include "kernels.h"
#include "stream_common.h"

namespace dsa {

namespace {

constexpr int kCeilWaves = 4;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Two full-entropy bf16 values per word: random sign and mantissa, exponent
// 2^-7 .. 2^0 (the magnitudes of unit-variance data scaled by 1/sqrt(128)).
__device__ __forceinline__ uint32_t bf16_pair(uint32_t r) {
  return (r & 0x807f807fu) | 0x3c003c00u | ((r >> 4) & 0x03800380u);
}
// Four e4m3 codes per word: random sign and mantissa, exponent field 4..11
// (never the NaN code).
__device__ __forceinline__ uint32_t e4m3_quad(uint32_t r) {
  const uint32_t e = ((r >> 3) & 0x07070707u) + 0x04040404u;
  return (r & 0x87878787u) | (e << 3);
}

template <int DT>
__device__ __forceinline__ u32x4 synth16(uint32_t seed) {
  u32x4 v;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t r = mix32(seed * 4u + (uint32_t)c);
    v[c] = DT == kBF16 ? bf16_pair(r) : e4m3_quad(r);
  }
  return v;
}

template <int DT, int MODE>
__global__ __launch_bounds__(kCeilWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mfma_ceiling(
    float* __restrict__ out, int iters) {
  using Tile = DirectTile<DT, 16384, kCeilWaves>;
  constexpr int RB = Frag<DT>::kRowBytes;
  constexpr int CPR = RB / 16;
  __shared__ u32x4 tile[64 * (CPR + 1)];
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t wseed = (uint32_t)(blockIdx.x * kCeilWaves + (tid >> 6)) * 0x10001u;
  for (int i = tid; i < 64 * (CPR + 1); i += kCeilWaves * 64) tile[i] = synth16<DT>(0x9e3779b9u + (uint32_t)i);

  // the wave's query: 64 head rows as two A fragments, and its head weights
  QuerySide<DT> qs;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int i = 0; i < Frag<DT>::kSteps; ++i) {
      const uint32_t s = wseed + (uint32_t)(((blk * 8 + i) * 64 + lane) * 2);
      if constexpr (DT == kBF16) {
        qs.a[blk].v[i] = synth16<DT>(s);
      } else {
        const u32x4 lo = synth16<DT>(s), hi = synth16<DT>(s + 1u);
        qs.a[blk].v[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      qs.wl[blk][v] = (float)(int)(mix32(wseed + 0x51u * (uint32_t)(blk * 16 + v) + (uint32_t)lane) & 0xffffu) *
                          (1.0f / 32768.0f) - 1.0f;
  __syncthreads();

  const int lk = lane & 31;
  Frag<DT> f;
  Tile::frag(f, tile, lk, lane);
  f32x16 acc[2][2];
  acc[0][0] = acc[0][1] = acc[1][0] = acc[1][1] = zero16();
  float tot = 0.0f;
  // mode 2: the linear row's A operand (rows 0, 1 of a 16-row block; lane l
  // holds row l % 16, dims 8 (l / 16) .. + 8 of each 32-dim k-step)
  bf16x8 ua[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 v = (lane & 15) < 2 ? synth16<kBF16>(wseed + 0x777u + (uint32_t)(ks * 64 + lane)) : u32x4{0u, 0u, 0u, 0u};
    ua[ks] = __builtin_bit_cast(bf16x8, v);
  }
  for (int it = 0; it + 1 < iters; it += 2) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int nkey = 32 * (sub ^ 1) + lk;  // the tile's other block next
      if constexpr (MODE == 0) {
#pragma unroll
        for (int i = 0; i < Frag<DT>::kSteps; ++i) {
          acc[sub][0] = mma_step<DT>(qs.a[0], f, i, acc[sub][0]);
          acc[sub][1] = mma_step<DT>(qs.a[1], f, i, acc[sub][1]);
          Tile::frag_step(f, tile, nkey, i, lane);
        }
      } else if constexpr (MODE == 2) {
        // the |x| form: 16 MFMAs interleaved with one abs-FMA per head and
        // key of the previous block, then the linear row of this block
        const f32x16& p0 = acc[sub ^ 1][0];
        const f32x16& p1 = acc[sub ^ 1][1];
        acc[sub][0] = zero16();
        acc[sub][1] = zero16();
        float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 2 * Frag<DT>::kSteps; ++m) {
          if ((m & 1) == 0) {
            acc[sub][0] = mma_step<DT>(qs.a[0], f, m >> 1, acc[sub][0]);
          } else {
            acc[sub][1] = mma_step<DT>(qs.a[1], f, m >> 1, acc[sub][1]);
            Tile::frag_step(f, tile, nkey, m >> 1, lane);
          }
#pragma unroll
          for (int u = 2 * m; u < 2 * m + 2; ++u) {
            const int e = u >> 2, g = u & 3;
            const float x = e < 4 ? p0[4 * g + e] : p1[4 * g + e - 4];
            const float wv = e < 4 ? qs.wl[0][4 * g + e] : qs.wl[1][4 * g + e - 4];
            c[g] = __builtin_fmaf(__builtin_fabsf(x), wv, c[g]);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (m & 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        // the linear row: keys 16 h + l % 16 of this block, dims 32 ks + 8 (l / 16)
        const int kb = 32 * (sub & 1);
        f32x4 lin[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          lin[h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const u32x4 kf = tile[(kb + 16 * h + (lane & 15)) * (CPR + 1) + 4 * ks + (lane >> 4)];
            lin[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua[ks], __builtin_bit_cast(bf16x8, kf), lin[h], 0, 0, 0);
          }
        }
        // rows 0 and 1 (lanes 0..15, v = 0, 1) to the lanes of key l % 32
        const float l0 = lin[0][0] + lin[0][1], l1 = lin[1][0] + lin[1][1];
        const int src = lane & 15;
        const float a0 = __shfl(l0, src, 64), a1 = __shfl(l1, src, 64);
        const float lk_term = (lane & 16) ? a1 : a0;
        tot += combine_single((c[0] + c[1]) + (c[2] + c[3])) + lk_term;
      } else {
        tot += combine_single(pipelined_partial<DT>(qs, f, acc[sub ^ 1][0], acc[sub ^ 1][1], acc[sub][0],
                                                    acc[sub][1],
                                                    [&](int i) { Tile::frag_step(f, tile, nkey, i, lane); }));
      }
    }
  }
  float r = tot;
#pragma unroll
  for (int e = 0; e < 16; ++e) r += acc[0][0][e] + acc[0][1][e] + acc[1][0][e] + acc[1][1][e];
  out[(size_t)blockIdx.x * (kCeilWaves * 64) + tid] = r;
}

}  // namespace

int mfma_ceiling_workgroups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -1;
  return 2 * cus;
}

hipError_t launch_mfma_ceiling(int dtype, int mode, int iters, int workgroups, float* out, hipStream_t st) {
  const dim3 grid(workgroups), block(kCeilWaves * 64);
  if (dtype == kBF16) {
    if (mode == 0)
      hipLaunchKernelGGL((k_mfma_ceiling<kBF16, 0>), grid, block, 0, st, out, iters);
    else if (mode == 1)
      hipLaunchKernelGGL((k_mfma_ceiling<kBF16, 1>), grid, block, 0, st, out, iters);
    else
      hipLaunchKernelGGL((k_mfma_ceiling<kBF16, 2>), grid, block, 0, st, out, iters);
  } else {
    if (mode == 0)
      hipLaunchKernelGGL((k_mfma_ceiling<kFP8, 0>), grid, block, 0, st, out, iters);
    else
      hipLaunchKernelGGL((k_mfma_ceiling<kFP8, 1>), grid, block, 0, st, out, iters);
  }
  return hipGetLastError();
}

}  // namespace dsa
