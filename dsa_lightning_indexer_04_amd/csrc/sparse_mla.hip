// sparse_mla.hip -- MLA core attention (MQA mode) over the indexer's selected
// positions.
//
// DeepSeek DSA FLOPs notes, section "Core Sparse Attention FLOPs": for query
// row t and its selected positions S_t, every one of the h = 128 heads scores
// the shared cache rows [C^KV | K^R] (512 + 64 values) with its query
// [Q^A | Q^R], a softmax over the selected positions gives P, and the output
// is Z = P C^KV_S (h x 512).  The softmax is taken of sm_scale * score.
//
// One workgroup per query row, 4 waves, 32 heads per wave.  Per tile of 32
// selected positions:
//   * the 32 cache rows are gathered straight from HBM into LDS (one 16-byte
//     chunk per lane, key-major, one pad chunk per row so column reads are
//     conflict-free), double-buffered: the next tile's rows load while this
//     tile is computed;
//   * S^T = K Q^T as a 32 keys x 32 heads MFMA block (36 k-steps of
//     32x32x16 bf16; the wave's 32 x 576 query block stays in registers), so
//     a lane owns one head: the softmax statistics are lane-local plus one
//     cross-half exchange;
//   * O^T += V^T P^T over the 16 blocks of 32 latent dims: P^T is taken from
//     the S^T accumulators as they lie (the contraction runs over the keys in
//     the order a lane's accumulator holds them), and the V^T operand is read
//     straight from the key-major tile with transposing LDS reads
//     (ds_read_b64_tr_b16: in each group of 16 lanes, lane 4r+q supplies 4
//     consecutive values of row r and lane c receives value c of each of the
//     4 rows -- here 4 keys of one latent dim).
// Softmax reference: each head subtracts a fixed reference (its first
// selected tile's maximum) instead of a running maximum, so the accumulators
// are never rescaled (a rescale, like any loop restart, makes the register
// allocator spill the query block).  The softmax does not depend on the
// constant subtracted; weights stay below 2^32 as long as no later score
// exceeds the reference by more than 32 (log2 units).  A row where one does
// is flagged together with its heads' true maxima, and a second launch of the
// kernel recomputes just the flagged rows with those maxima as references
// (no weight above 1).  Scores of ordinary range never flag a row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>

#include "kernels.h"

namespace dsa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kHeads = 128;
constexpr int kDc = 512;           // latent dims
constexpr int kDr = 64;            // RoPE dims
constexpr int kRow = kDc + kDr;    // values per cache row / query head
constexpr int kChunks = kRow / 8;  // 16-byte chunks per row (72)
constexpr int kSlots = kChunks + 1;  // LDS slots per key row (one pad)
constexpr int kTile = 32;          // selected positions per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// one direct-load instruction fills 1 KiB (64 lanes x 16 B); each wave
// issues the same number of them per tile, so the buffer holds
// kWaves * ceil(37 / kWaves) KiB and the slots past the tile land in it
constexpr int kLoadsPerWave = (kTile * kSlots * 16 / 1024 + 1 + kWaves - 1) / kWaves;  // 10
constexpr int kKtBytes = kWaves * kLoadsPerWave * 1024;                                // 40960
constexpr int kKSteps = kRow / 16;             // 36
constexpr int kMaxTopk = 2048;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRestartMargin = 32.0f;
constexpr int kMaxSplits = 8;
constexpr int kAhead = 6;  // LDS operand reads in flight per MFMA chain

constexpr int kOBlocks = kDc / 32;  // 32-dim output blocks per head group

template <int kBufs>
struct Smem {
  uint8_t kt[kBufs][kKtBytes];
  int32_t idx[kMaxTopk];
  int32_t last[kWaves];
  int32_t vote[kWaves];  // a wave saw a score above its reference + margin
};

// kRetry = false: first pass over every row; true: recompute the rows the
// first pass flagged, with the recorded maxima as references.
// kSplit: each workgroup takes one of nsplit consecutive ranges of a row's
// tiles (few rows, e.g. decode) and writes fp32 partial results (unnormalised
// output, reference maximum, weight sum) that k_mla_merge combines.
template <bool kRetry, bool kSplit>
__global__ __launch_bounds__(kThreads, 1) void k_sparse_mla(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ kv,
                                                            const int32_t* __restrict__ indices, int Q, int N,
                                                            int topk, const int32_t* __restrict__ page_table,
                                                            int page_size, int pages_per_seq, int num_pages,
                                                            float scale_log2, uint16_t* __restrict__ out,
                                                            float* __restrict__ lse, float* __restrict__ row_max,
                                                            int32_t* __restrict__ retry, int nsplit,
                                                            float* __restrict__ part_o, float* __restrict__ part_ml) {
  // one work unit: a row, or (kSplit) a row's tile range
  const size_t unit = blockIdx.x;
  if (kRetry && retry[unit] == 0) return;  // uniform over the workgroup
  __shared__ Smem<2> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t row = kSplit ? unit / nsplit : unit;  // b * Q + t
  const int split = kSplit ? (int)(unit % nsplit) : 0;
  const size_t b = row / (size_t)Q;
  // flat layout: the sequence's rows; paged: the pool, rows addressed through the table
  const uint16_t* kvb = page_table ? kv : kv + b * (size_t)N * kRow;
  const int32_t* ptab = page_table ? page_table + b * (size_t)pages_per_seq : nullptr;

  // ---- selected positions of the row: LDS copy of their cache rows (-1 past
  // topk or out of range)
  const int32_t* irow = indices + row * (size_t)topk;
  int last = -1;
  for (int i = tid; i < kMaxTopk; i += kThreads) {
    int v = -1;
    if (i < topk) {
      v = irow[i];
      if (v < 0 || v >= N) v = -1;
      if (v >= 0 && ptab) {
        const int pg = min(max(ptab[v / page_size], 0), num_pages - 1);
        v = pg * page_size + v % page_size;
      }
    }
    sm.idx[i] = v;
    if (v >= 0) last = i;
  }
  // the last valid entry bounds the tiles to visit
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (lane == 0) {
    sm.last[wave] = last;
    sm.vote[wave] = 0;
  }

  // ---- this wave's 32 heads of the query row as MFMA B operands (Q^T):
  // lane l holds head l%32, dims 16kk + 8(l/32) .. +7 for k-step kk
  const uint16_t* qh = q + (row * kHeads + wave * 32 + l32) * kRow + 8 * half;
  u32x4 qf[kKSteps];
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) qf[kk] = *reinterpret_cast<const u32x4*>(qh + 16 * kk);
  __syncthreads();
  const int lastv = max(max(sm.last[0], sm.last[1]), max(sm.last[2], sm.last[3]));
  const int ntiles = (lastv + kTile) / kTile;  // 0 when nothing is selected

  // ---- gather of one tile into kt[buf]: slot s of the tile (key s/73, chunk
  // s%73) is lane s%64 of load instruction s/64; wave w issues instructions
  // w, w+4, ... (kLoadsPerWave of them), each filling 1 KiB of LDS.  Pad
  // slots (chunk 72) and slots past the tile re-read a chunk of the tile;
  // invalid entries read row 0 (their scores are masked).  A cursor walks
  // this lane's slots: consecutive instructions of a wave are 256 slots apart
  // (3 rows of 73 plus 37), so no division per load.
  struct Cursor {
    int key, c;
  };
  auto cursor0 = [&]() {
    const int s0 = wave * 64 + lane;
    return Cursor{s0 / kSlots, s0 - (s0 / kSlots) * kSlots};
  };
  auto issue_one = [&](int tile, int buf, int i, Cursor& cur) {
    const int j = wave + kWaves * i;
    const bool past = cur.key >= kTile;
    const int key = past ? kTile - 1 : cur.key;
    const int c = (past || cur.c == kChunks) ? 0 : cur.c;
    const int pos = max(sm.idx[tile * kTile + key], 0);
    const uint16_t* src = kvb + (size_t)pos * kRow + 8 * c;
    __builtin_amdgcn_global_load_lds(src, reinterpret_cast<uint32_t*>(&sm.kt[buf][j * 1024]), 16, 0, 0);
    cur.c += kWaves * 64 - 3 * kSlots;
    cur.key += 3;
    if (cur.c >= kSlots) cur.c -= kSlots, cur.key += 1;
  };
  auto issue_tile = [&](int tile, int buf) {
    Cursor cur = cursor0();
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) issue_one(tile, buf, i, cur);
  };

  // O^T accumulators: 16 blocks of 32 latent dims x 32 heads (256 registers)
  f32x16 o[kOBlocks];
#pragma unroll
  for (int i = 0; i < kOBlocks; ++i) o[i] = f32x16{0};
  const int head = wave * 32 + l32;
  float m_ref = kRetry ? row_max[unit * kHeads + head] : -INFINITY;
  float m_seen = -INFINITY, l_run = 0.0f;
  bool over = false;  // a score exceeded the reference by more than the margin

  // this unit's tiles
  int t0 = 0, t1 = ntiles;
  if (kSplit) {
    const int per = (ntiles + nsplit - 1) / nsplit;
    t0 = min(ntiles, split * per);
    t1 = min(ntiles, t0 + per);
  }
  if (t0 < t1) issue_tile(t0, 0);
  for (int tile = t0; tile < t1; ++tile) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the tile have landed
    __syncthreads();
    const int buf = (tile - t0) & 1;
    // the next tile's rows load into the other buffer during this whole tile
    // (interleaved with the score MFMAs below); that buffer's last readers
    // finished before the barrier above.  The last tile re-reads itself into
    // the idle buffer.
    const int nt = tile + 1 < t1 ? tile + 1 : tile;
    Cursor cur = cursor0();

    // ---- S^T = K Q^T (32 keys x 32 heads); operands read kAhead k-steps
    // ahead.  The fenced steps also carry the next tile's gather (one load
    // every third step): the MFMAs run while these issue.
    f32x16 s = f32x16{0};
    const uint8_t* ka = &sm.kt[buf][(l32 * kSlots + half) * 16];
    {
      u32x4 ar[kAhead];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kAhead; ++i) ar[i] = *reinterpret_cast<const u32x4*>(ka + i * 32);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ar[kk % kAhead]),
                                                    __builtin_bit_cast(bf16x8, qf[kk]), s, 0, 0, 0);
        if (kk + kAhead < kKSteps) ar[kk % kAhead] = *reinterpret_cast<const u32x4*>(ka + (kk + kAhead) * 32);
        if (kk % 3 == 1 && kk / 3 < kLoadsPerWave) issue_one(nt, buf ^ 1, kk / 3, cur);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- online softmax per head (lane l%32), base 2
    // lane holds keys 8(v/4) + 4*half + v%4 of the tile; bit r of `valid`
    // says whether the tile's key r is a selected position
    const uint32_t valid = (uint32_t)__builtin_amdgcn_ballot_w64(sm.idx[tile * kTile + l32] >= 0);
    float sv[16];
    float mx = -INFINITY;
    if (valid == 0xFFFFFFFFu) {  // uniform: every key of the tile selected (all but a row's last tile)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sv[v] = s[v] * scale_log2;
        mx = fmaxf(mx, sv[v]);
      }
    } else {
      const uint32_t mine = valid >> (4 * half);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool ok = (mine >> (8 * (v >> 2) + (v & 3))) & 1u;
        sv[v] = ok ? s[v] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[v]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (!kRetry) {
      m_seen = fmaxf(m_seen, mx);
      if (m_ref == -INFINITY) m_ref = mx;  // first selected tile (nothing accumulated yet)
      over |= mx > m_ref + kRestartMargin;
    }
    // weights; a head with nothing selected yet keeps m_ref = -inf and weights 0
    const float msub = m_ref == -INFINITY ? 0.0f : m_ref;
    auto weights = [&](int g, int j, uint32_t& w) {
      const float p0 = __builtin_amdgcn_exp2f(sv[8 * g + 2 * j] - msub);
      const float p1 = __builtin_amdgcn_exp2f(sv[8 * g + 2 * j + 1] - msub);
      l_run += p0 + p1;
      const __bf16 h0 = static_cast<__bf16>(p0), h1 = static_cast<__bf16>(p1);
      w = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    };
    u32x4 pb[2];
    {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) weights(0, j, w[j]);
      pb[0] = u32x4{w[0], w[1], w[2], w[3]};
    }
    // ---- O^T += V^T P^T: 16 blocks of 32 latent dims, 2 k-steps of 16 keys
    // (k-step outer, so consecutive MFMAs update different blocks).  The
    // operand of lane l (latent dim 32 blk + l%32, k-half h = l/32) is keys
    // 16 g + 4h + 0..3 and 16 g + 8 + 4h + 0..3 of that dim: two transposing
    // reads, in which lane 4r+q of each 16-lane group supplies dims
    // 16 (group%2) + 4q .. +3 of key 16 g + 4h + r (+8).  Read kAhead steps ahead.
    {
      const int grp = lane >> 4, r = (lane >> 2) & 3, qd = lane & 3;
      uint32_t vb = (uint32_t)(buf * kKtBytes + (4 * (grp >> 1) + r) * kSlots * 16 + (16 * (grp & 1) + 4 * qd) * 2);
      asm volatile("" : "+v"(vb));
      const uint8_t* vbase = reinterpret_cast<const uint8_t*>(sm.kt) + vb;
      auto vread = [&](int st) {
        const int blk = st % kOBlocks, g = st / kOBlocks;
        const uint8_t* a0 = vbase + 16 * g * kSlots * 16 + 64 * blk;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(a0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(a0 + 8 * kSlots * 16));
        return u32x4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                     (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                     (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                     (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
      };
      constexpr int kSteps = 2 * kOBlocks;
      u32x4 ar[kAhead];
      uint32_t w1[4];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kAhead; ++i) ar[i] = vread(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const int blk = st % kOBlocks, g = st / kOBlocks;
        if (st == kOBlocks) pb[1] = u32x4{w1[0], w1[1], w1[2], w1[3]};
        o[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ar[st % kAhead]),
                                                         __builtin_bit_cast(bf16x8, pb[g]), o[blk], 0, 0, 0);
        if (st + kAhead < kSteps) ar[st % kAhead] = vread(st + kAhead);
        if (st < 4) weights(1, st, w1[st]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // the last tile's redundant loads into the idle buffer must land before
  // the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0);

  // ---- normalise and write: lane holds head l%32 and, per block, dims
  // 32 blk + 8(v/4) + 4 half + v%4
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (!kRetry) {
    // flag the row if any head saw a score too far above its reference, and
    // record every head's maximum for the second pass
    const bool w_over = __builtin_amdgcn_ballot_w64(over) != 0;
    if (lane == 0) sm.vote[wave] = w_over;
    __syncthreads();
    if (tid == 0) retry[unit] = sm.vote[0] | sm.vote[1] | sm.vote[2] | sm.vote[3];
    if (half == 0) row_max[unit * kHeads + head] = m_seen;
  }
  if (kSplit) {
    // partial results: the unnormalised output, the reference and the weight sum
    float* prow = part_o + (unit * kHeads + head) * kDc;
#pragma unroll
    for (int blk = 0; blk < kOBlocks; ++blk) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(prow + 32 * blk + 8 * g + 4 * half) =
            make_float4(o[blk][4 * g], o[blk][4 * g + 1], o[blk][4 * g + 2], o[blk][4 * g + 3]);
    }
    if (half == 0) *reinterpret_cast<float2*>(part_ml + (unit * kHeads + head) * 2) = make_float2(m_ref, l_tot);
    return;
  }
  uint16_t* orow = out + (row * kHeads + head) * kDc;
  auto store_block = [&](int blk, const f32x16& acc) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const __bf16 h0 = static_cast<__bf16>(acc[4 * g + 2 * j] * inv);
        const __bf16 h1 = static_cast<__bf16>(acc[4 * g + 2 * j + 1] * inv);
        w[j] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      }
      *reinterpret_cast<uint2*>(orow + 32 * blk + 8 * g + 4 * half) = make_uint2(w[0], w[1]);
    }
  };
#pragma unroll
  for (int blk = 0; blk < kOBlocks; ++blk) store_block(blk, o[blk]);
  if (lse && half == 0)
    lse[row * kHeads + head] = l_tot > 0.0f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// Combines a row's nsplit partial results: with M the largest reference of
// the splits that saw a selected position, weights 2^(m_s - M), the output is
// sum_s w_s O_s / sum_s w_s l_s and the log-sum-exp (M + log2 sum_s w_s l_s) ln 2.
// Each workgroup takes two heads of one row; a thread takes 4 latent dims.
__global__ __launch_bounds__(256) void k_mla_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                   int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse) {
  const size_t row = blockIdx.x / (kHeads / 2);
  const int head = (int)(blockIdx.x % (kHeads / 2)) * 2 + (threadIdx.x >> 7);
  const int d = (threadIdx.x & 127) * 4;
  float2 ml[kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    ml[sp] = sp < nsplit ? *reinterpret_cast<const float2*>(part_ml + ((row * nsplit + sp) * kHeads + head) * 2)
                         : make_float2(-INFINITY, 0.0f);
  float mmax = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (ml[sp].y > 0.0f) mmax = fmaxf(mmax, ml[sp].x);
  float wsum = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp) {
    if (sp >= nsplit) break;
    const float w = ml[sp].y > 0.0f ? __builtin_amdgcn_exp2f(ml[sp].x - mmax) : 0.0f;
    wsum += w * ml[sp].y;
    const float4 v = *reinterpret_cast<const float4*>(part_o + ((row * nsplit + sp) * kHeads + head) * kDc + d);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const __bf16 h0 = static_cast<__bf16>(acc.x * inv), h1 = static_cast<__bf16>(acc.y * inv);
  const __bf16 h2 = static_cast<__bf16>(acc.z * inv), h3 = static_cast<__bf16>(acc.w * inv);
  *reinterpret_cast<uint2*>(out + (row * kHeads + head) * kDc + d) =
      make_uint2((uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16),
                 (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16));
  if (lse && (threadIdx.x & 127) == 0)
    lse[row * kHeads + head] = wsum > 0.0f ? (mmax + __log2f(wsum)) * kLn2 : -INFINITY;
}

}  // namespace

int mla_splits(int rows, int requested) {
  if (requested > 0) return min(requested, kMaxSplits);
  return rows < 256 ? min(kMaxSplits, (512 + rows - 1) / rows) : 1;
}

hipError_t launch_sparse_mla(const MlaProblem& p, float sm_scale, uint16_t* out, float* lse, float* row_max,
                             int32_t* retry, int nsplit, float* part_o, float* part_ml, hipStream_t st) {
  const size_t rows = (size_t)p.B * p.Q;
  const dim3 grid((unsigned)(rows * nsplit)), block(kThreads);
  const float sl = sm_scale * kLog2e;
  auto run = [&](auto first, auto again) {
    int slot = prof_open("k_sparse_mla", st);
    hipLaunchKernelGGL(first, grid, block, 0, st, p.q, p.kv, p.indices, p.Q, p.N, p.topk, p.page_table, p.page_size,
                       p.pages_per_seq, p.num_pages, sl, out, lse, row_max, retry, nsplit, part_o, part_ml);
    prof_close(slot, st);
    slot = prof_open("k_sparse_mla_retry", st);
    hipLaunchKernelGGL(again, grid, block, 0, st, p.q, p.kv, p.indices, p.Q, p.N, p.topk, p.page_table, p.page_size,
                       p.pages_per_seq, p.num_pages, sl, out, lse, row_max, retry, nsplit, part_o, part_ml);
    prof_close(slot, st);
  };
  if (nsplit > 1) {
    run(k_sparse_mla<false, true>, k_sparse_mla<true, true>);
    const int slot = prof_open("k_mla_merge", st);
    hipLaunchKernelGGL(k_mla_merge, dim3((unsigned)(rows * (kHeads / 2))), dim3(256), 0, st, part_o, part_ml, nsplit,
                       out, lse);
    prof_close(slot, st);
  } else {
    run(k_sparse_mla<false, false>, k_sparse_mla<true, false>);
  }
  return hipGetLastError();
}

}  // namespace dsa
