// score_tile.h -- the one device routine that scores (query, key) pairs.
//
// Index score (DeepSeek DSA FLOPs notes, section "Lightning Indexer FLOPs",
// the index-score equation):  I[t,s] = sum_j w[t,j] ReLU(q[t,j,:] . k[s,:]),
// 64 heads of 128, one key row shared by every head.
//
// Every path of the library (full score matrix, streaming Top-K, seed
// rescoring, survivor refinement) computes a pair's score with the code in
// this file, so a pair's fp32 score is bit-identical whichever path, tile or
// column position produced it.  That is what lets the pruned Top-K return
// exactly the unpruned index set.
//
// MFMA mapping (gfx950, wave64):
//   rows (M) = heads: two 32-row blocks per query (heads 0..31, 32..63)
//   cols (N) = 32 keys
//   K        = the 128 feature dims.  Both operands use the same lane->dim
//              permutation: k-step i takes dims 16i..16i+15 (fp8: 64i..
//              64i+63), lane l (half h = l/32) the lower or upper half of
//              them, so the two lanes that feed one row in a step read
//              adjacent 16 (fp8: 32) bytes of it.
// bf16: v_mfma_f32_32x32x16_bf16, 8 k-steps of 16 (lane: 8 dims per step).
// fp8 : v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales, 2 k-steps of 64
//       (lane: 32 dims per step), OCP e4m3 operands.
// Accumulator layout (32x32 blocks): lane l, register v holds
//   row 8*(v/4) + 4*(l/32) + (v%4), column l%32.
// So each lane holds 16 heads of each block for one key; the head sum is
// lane-local over 32 heads, then one cross-half exchange adds the other 32.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace dsa {

constexpr int kHeads = 64;
constexpr int kDim = 128;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

enum : int { kBF16 = 0, kFP8 = 1 };

template <int DT>
struct Frag;  // per-lane operand fragment of one 32-row (or 32-key) block, K = 128

template <>
struct Frag<kBF16> {
  static constexpr int kSteps = 8;        // 8 x (32x32x16)
  static constexpr int kRowBytes = 256;   // 128 bf16
  static constexpr int kLaneBytes = 128;  // bytes one lane feeds over the k-steps
  u32x4 v[8];
};

template <>
struct Frag<kFP8> {
  static constexpr int kSteps = 2;        // 2 x (32x32x64)
  static constexpr int kRowBytes = 128;   // 128 e4m3 codes
  static constexpr int kLaneBytes = 64;
  i32x8 v[2];
};

// Load one lane's fragment of a row (query head row or key row) from any
// address space: `row` points at the start of the row (kRowBytes long).
// Step i of half h is 16-byte chunk 2i + h (bf16), chunks 4i + 2h and
// 4i + 2h + 1 (fp8).
template <int DT>
__device__ __forceinline__ void load_frag(Frag<DT>& f, const uint8_t* row, int lane) {
  if constexpr (DT == kBF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row) + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = p[2 * i];
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(row) + 2 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 lo = p[4 * i], hi = p[4 * i + 1];
      f.v[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }
}

// Wait for every outstanding vector-memory load of this wave (s_waitcnt
// vmcnt(0), other counters untouched).  Issued once after the loop-invariant
// loads (query fragments, weights): without it the compiler cannot tell at
// the loop head that they have landed and waits for vmcnt(0) inside the key
// loop, which also waits for the next tile's prefetch.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// One k-step of a 32x32 block: acc += A(32 rows) x B(32 keys)^T over the
// step's slice of the 128 dims.
template <int DT>
__device__ __forceinline__ f32x16 mma_step(const Frag<DT>& a, const Frag<DT>& b, int i, f32x16 acc) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v[i]), __builtin_bit_cast(bf16x8, b.v[i]),
                                                   acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v[i], b.v[i], acc, 0, 0, 0, 127, 0, 127);
}

// acc += A(32 rows) x B(32 keys)^T over K = 128.
template <int DT>
__device__ __forceinline__ f32x16 mma_block(const Frag<DT>& a, const Frag<DT>& b, f32x16 acc) {
#pragma unroll
  for (int i = 0; i < Frag<DT>::kSteps; ++i) acc = mma_step<DT>(a, b, i, acc);
  return acc;
}

// The query side of a score: 64 head rows as two A fragments plus this
// lane's 32 head weights, wl[blk][v] = w[32*blk + 8*(v/4) + 4*(lane/32) + v%4].
template <int DT>
struct QuerySide {
  Frag<DT> a[2];
  float wl[2][16];
};

// q_heads: the query's [64][128] rows; w_row: its 64 weights.
template <int DT>
__device__ __forceinline__ void load_query(QuerySide<DT>& qs, const uint8_t* q_heads, const float* w_row,
                                           int lane) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
    load_frag<DT>(qs.a[blk], q_heads + (size_t)(32 * blk + r) * Frag<DT>::kRowBytes, lane);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int v = 0; v < 16; ++v) qs.wl[blk][v] = w_row[32 * blk + 8 * (v >> 2) + 4 * h + (v & 3)];
}

// ReLU of a finite fp32 value as one integer max on its bits: non-negative
// floats are non-negative int32 patterns, negative floats (and -0) negative
// ones, so max(bits, 0) is the bit pattern of max(x, +0).  (fmaxf would add
// a NaN-canonicalising max per element.)
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// This lane's share of the head sum for its key column: 32 of the 64 heads,
// in a fixed order (four chains of eight, then a fixed pairing).
__device__ __forceinline__ float head_partial(const f32x16& s0, const f32x16& s1, const float (&wl)[2][16]) {
  float c[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(relu_bits(s0[4 * g + e]), wl[0][4 * g + e], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(relu_bits(s1[4 * g + e]), wl[1][4 * g + e], acc);
    c[g] = acc;
  }
  return (c[0] + c[1]) + (c[2] + c[3]);
}

// Head weights of this lane's 32 heads from a row of 64 weights (any address
// space): the same order as QuerySide::wl.
__device__ __forceinline__ void load_wl(float (&wl)[2][16], const float* w_row, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int v = 0; v < 16; ++v) wl[blk][v] = w_row[32 * blk + 8 * (v >> 2) + 4 * h + (v & 3)];
}

// head_partial with the weights read from a 64-float row four at a time
// (exactly the same FMA sequence, so the same bits).
__device__ __forceinline__ float head_partial_w(const f32x16& s0, const f32x16& s1, const float* w_row, int lane) {
  const int h = lane >> 5;
  float c[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 w0 = *reinterpret_cast<const float4*>(w_row + 8 * g + 4 * h);
    const float4 w1 = *reinterpret_cast<const float4*>(w_row + 32 + 8 * g + 4 * h);
    float acc = 0.0f;
    acc = __builtin_fmaf(relu_bits(s0[4 * g + 0]), w0.x, acc);
    acc = __builtin_fmaf(relu_bits(s0[4 * g + 1]), w0.y, acc);
    acc = __builtin_fmaf(relu_bits(s0[4 * g + 2]), w0.z, acc);
    acc = __builtin_fmaf(relu_bits(s0[4 * g + 3]), w0.w, acc);
    acc = __builtin_fmaf(relu_bits(s1[4 * g + 0]), w1.x, acc);
    acc = __builtin_fmaf(relu_bits(s1[4 * g + 1]), w1.y, acc);
    acc = __builtin_fmaf(relu_bits(s1[4 * g + 2]), w1.z, acc);
    acc = __builtin_fmaf(relu_bits(s1[4 * g + 3]), w1.w, acc);
    c[g] = acc;
  }
  return (c[0] + c[1]) + (c[2] + c[3]);
}

// Full-head partial for one query against one 32-key block, with the head
// weights read from a row of 64 floats (same arithmetic as query_partial).
template <int DT>
__device__ __forceinline__ float query_partial_w(const Frag<DT> (&a)[2], const Frag<DT>& kb, const float* w_row,
                                                 int lane) {
  f32x16 s0 = mma_block<DT>(a[0], kb, zero16());
  f32x16 s1 = mma_block<DT>(a[1], kb, zero16());
  return head_partial_w(s0, s1, w_row, lane);
}

// Full-head partial for one query against one 32-key block.
template <int DT>
__device__ __forceinline__ float query_partial(const QuerySide<DT>& qs, const Frag<DT>& kb) {
  f32x16 s0 = mma_block<DT>(qs.a[0], kb, zero16());
  f32x16 s1 = mma_block<DT>(qs.a[1], kb, zero16());
  return head_partial(s0, s1, qs.wl);
}

// One software-pipelined step of a key scan: the MFMAs of a new 32-key block
// (into n0/n1, the same k-step sequence as mma_block from zero) issued one by
// one, each followed by its share of the previous block's head sum (p0/p1),
// so one wave keeps the matrix core and the vector ALU busy together.  The
// head sum is head_partial's, operation for operation: chain g starts at +0
// and takes relu(p0[4g+e]) * wl[0][4g+e] for e = 0..3, then the same over
// p1 and wl[1]; only the four chains are interleaved with each other.
// Rolling operand prefetch: once both MFMAs of k-step i have been issued,
// step i of kb is dead and `next(i)` reloads it with step i of the next
// block's key fragment, so the LDS reads of block j+1 run under block j's
// MFMAs and no MFMA waits on a fresh LDS read.
template <int DT, class Next>
__device__ __forceinline__ float pipelined_partial(const QuerySide<DT>& qs, Frag<DT>& kb, const f32x16& p0,
                                                   const f32x16& p1, f32x16& n0, f32x16& n1, Next&& next) {
  constexpr int kMfma = 2 * Frag<DT>::kSteps;
  constexpr int kUnits = 32 / kMfma;  // (relu, fma) pairs after each MFMA
  constexpr int kReads = Frag<DT>::kLaneBytes / 16 / Frag<DT>::kSteps;  // ds_read_b128 per k-step
  float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  n0 = zero16();
  n1 = zero16();
#pragma unroll
  for (int m = 0; m < kMfma; ++m) {
    if ((m & 1) == 0) {
      n0 = mma_step<DT>(qs.a[0], kb, m >> 1, n0);
    } else {
      n1 = mma_step<DT>(qs.a[1], kb, m >> 1, n1);
      next(m >> 1);
    }
#pragma unroll
    for (int u = m * kUnits; u < (m + 1) * kUnits; ++u) {
      const int e = u >> 2, g = u & 3;
      const float x = e < 4 ? p0[4 * g + e] : p1[4 * g + e - 4];
      const float wv = e < 4 ? qs.wl[0][4 * g + e] : qs.wl[1][4 * g + e - 4];
      c[g] = __builtin_fmaf(relu_bits(x), wv, c[g]);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // this MFMA
    if (m & 1) __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // the freed step's reload
    __builtin_amdgcn_sched_group_barrier(0x002, 2 * kUnits, 0);  // then its VALU share
  }
  return (c[0] + c[1]) + (c[2] + c[3]);
}

// Cross-half sum through an LDS permute: the same bits as combine_swap.
// Kernels whose MFMA/VALU interleave is steered by scheduling groups use
// this form: the scheduler does not group around the inline asm of the swap.
__device__ __forceinline__ float combine_single(float p) { return p + __shfl_xor(p, 32, 64); }

// Cross-half sum: lanes l and l^32 hold the two halves (heads with row/4
// even / odd) of the same key column's head sum; every lane gets p[l] +
// p[l^32].  One v_permlane32_swap of two copies of p leaves lanes 0..31 of
// the first copy and lanes 32..63 of the second unchanged and swaps the
// other halves, so first + second is the pair sum in every lane (fp32
// addition is commutative: the same bits in both lanes of a pair, and in
// every path).  Written in inline asm because this compiler folds the two
// results of the permlane32 swap builtin into one; the s_nop pairs keep two
// wait states on both sides of the swap.  A VALU swap instead of an LDS
// permute keeps the exchange off the LDS queue.
__device__ __forceinline__ float combine_swap(float p) {
  float a = p, b = p;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}

// The lane exchange of combine_swap on two values: afterwards a holds
// (a[0..31], b[0..31]) and b holds (a[32..63], b[32..63]).
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// Dequantisation of fp8 scores: (q_scale * k_scale) * head_sum, same order everywhere.
__device__ __forceinline__ float apply_scales(float sum, float qscale, float kscale) {
  return sum * (qscale * kscale);
}

// Monotone 32-bit code of a finite fp32 score (larger score -> larger code);
// -0 maps like +0.
__device__ __forceinline__ uint32_t mono_code(float s) {
  uint32_t u = __builtin_bit_cast(uint32_t, s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float mono_decode(uint32_t c) {
  uint32_t u = (c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c;
  return __builtin_bit_cast(float, u);
}
// 64-bit record: larger record = larger score, then smaller key index.
__device__ __forceinline__ uint64_t make_record(float s, uint32_t key) {
  return ((uint64_t)mono_code(s) << 32) | (uint64_t)(0xFFFFFFFFu - key);
}
__device__ __forceinline__ uint32_t record_key(uint64_t r) { return 0xFFFFFFFFu - (uint32_t)r; }
__device__ __forceinline__ float record_score(uint64_t r) { return mono_decode((uint32_t)(r >> 32)); }

// A float that every score whose record is >= thr reaches (s >= it), for a
// cheap pre-test before building records: the decoded high half of thr, or
// -inf when that half lies below every finite score's code.
__device__ __forceinline__ float record_floor(uint64_t thr) {
  const uint32_t c = (uint32_t)(thr >> 32);
  return c < 0x00800000u ? -INFINITY : mono_decode(c);
}

}  // namespace dsa
