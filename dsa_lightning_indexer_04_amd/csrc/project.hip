// project.hip -- the indexer projections and the per-token output conversion.
//
// DeepSeek DSA FLOPs notes, section "Indexer projections": Q^I = C^Q W_IQ,
// K^I = X W_IK, W^I = X W_IW.  The products are plain bf16 GEMMs with fp32
// accumulation (rocBLAS, both operands K-contiguous).  They run per block of
// tokens into an fp32 staging buffer; k_proj_out then reads each token's
// 8192 + 192 fp32 outputs once and writes q/k in the requested dtype and w.
//
// Why a staging pass and not a GEMM epilogue: a token's one fp8 scale covers
// all 64 heads, so no code can be written before the whole 8192-wide row is
// known; a GEMM tile sees 128-256 columns.  The query GEMM and the output
// pass alternate over token blocks of 65536 tokens (2 GiB of fp32 staging),
// which bounds the workspace; smaller blocks were measured no faster (the
// staging is not kept in the Infinity Cache to any useful degree).  The thin
// key/weight GEMM runs once over all tokens.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include <cstdlib>
#include <string>
#include <unordered_map>

#include "kernels.h"

namespace dsa {
namespace {

constexpr int kQCols = 64 * 128;  // query outputs per token
constexpr int kKWCols = 128 + 64;  // key outputs, then head weights
constexpr int kOutThreads = 256;
constexpr float kFp8Max = 448.0f;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Scale and reciprocal of a row whose largest magnitude is amax.
__device__ __forceinline__ void fp8_scale(float amax, float* scale, float* inv) {
  const bool zero = !(amax > 0.0f);
  *scale = zero ? 1.0f : __fdiv_rn(amax, kFp8Max);
  *inv = zero ? 1.0f : __fdiv_rn(kFp8Max, amax);
}

// Four fp32 values -> four e4m3fn codes (x * inv, saturated, nearest even).
__device__ __forceinline__ uint32_t fp8x4(float4 v, float inv) {
  const float a = fminf(fmaxf(v.x * inv, -kFp8Max), kFp8Max);
  const float b = fminf(fmaxf(v.y * inv, -kFp8Max), kFp8Max);
  const float c = fminf(fmaxf(v.z * inv, -kFp8Max), kFp8Max);
  const float d = fminf(fmaxf(v.w * inv, -kFp8Max), kFp8Max);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ uint32_t fp8x2(float2 v, float inv) {
  const float a = fminf(fmaxf(v.x * inv, -kFp8Max), kFp8Max);
  const float b = fminf(fmaxf(v.y * inv, -kFp8Max), kFp8Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// One workgroup per token.  dq [T][8192] and dkw [T][192] fp32 staging rows.
// OUT: 0 = fp8 codes + scales, 1 = bf16, 2 = fp32.
template <int OUT>
__global__ __launch_bounds__(kOutThreads) void k_proj_out(const float* __restrict__ dq, const float* __restrict__ dkw,
                                                          uint8_t* __restrict__ q_out, float* __restrict__ q_scale,
                                                          uint8_t* __restrict__ k_out, float* __restrict__ k_scale,
                                                          float* __restrict__ w_out) {
  constexpr int kVec = kQCols / 4 / kOutThreads;  // float4 per thread (8)
  __shared__ float red[kOutThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t t = blockIdx.x;
  const f32x4* src = reinterpret_cast<const f32x4*>(dq + t * kQCols);
  float4 v[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const f32x4 x = __builtin_nontemporal_load(src + j * kOutThreads + tid);
    v[j] = make_float4(x[0], x[1], x[2], x[3]);
  }
  const float* kw = dkw + t * kKWCols;

  if constexpr (OUT == 0) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kVec; ++j)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    // the key row: wave 0, two values per lane
    if (wave == 0) {
      const float2 kv = *reinterpret_cast<const float2*>(kw + 2 * lane);
      const float km = wave_max(fmaxf(fabsf(kv.x), fabsf(kv.y)));
      float ks, kinv;
      fp8_scale(km, &ks, &kinv);
      reinterpret_cast<uint16_t*>(k_out + t * 128)[lane] = (uint16_t)fp8x2(kv, kinv);
      if (lane == 0) k_scale[t] = ks;
    }
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float qs, qinv;
    fp8_scale(amax, &qs, &qinv);
    uint32_t* dst = reinterpret_cast<uint32_t*>(q_out + t * kQCols);
#pragma unroll
    for (int j = 0; j < kVec; ++j) dst[j * kOutThreads + tid] = fp8x4(v[j], qinv);
    if (tid == 0) q_scale[t] = qs;
  } else if constexpr (OUT == 1) {
    uint2* dst = reinterpret_cast<uint2*>(q_out + t * kQCols * 2);
#pragma unroll
    for (int j = 0; j < kVec; ++j)
      dst[j * kOutThreads + tid] = make_uint2(bf16_rne(v[j].x) | (bf16_rne(v[j].y) << 16),
                                              bf16_rne(v[j].z) | (bf16_rne(v[j].w) << 16));
    if (wave == 0) {
      const float2 kv = *reinterpret_cast<const float2*>(kw + 2 * lane);
      reinterpret_cast<uint32_t*>(k_out + t * 128 * 2)[lane] = bf16_rne(kv.x) | (bf16_rne(kv.y) << 16);
    }
  } else {
    float4* dst = reinterpret_cast<float4*>(q_out + t * kQCols * 4);
#pragma unroll
    for (int j = 0; j < kVec; ++j) dst[j * kOutThreads + tid] = v[j];
    if (wave == 0)
      reinterpret_cast<float2*>(k_out + t * 128 * 4)[lane] = *reinterpret_cast<const float2*>(kw + 2 * lane);
  }
  // head weights: wave 1 copies the 64 fp32 values
  if (wave == 1) w_out[t * 64 + lane] = kw[128 + lane];
}

// ------------------------------------------------------------------ rocBLAS

const char* blas_name(rocblas_status s) { return rocblas_status_to_string(s); }

// One handle per thread and device (rocBLAS handles are not thread-safe).
// They live until the process ends.  Creating one allocates device memory,
// which a stream under graph capture cannot take: a first call on a
// capturing stream is refused (*unsupported set) instead.
rocblas_handle blas_handle(hipStream_t st, std::string* err, bool* unsupported) {
  thread_local std::unordered_map<int, rocblas_handle> handles;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *err = "hipGetDevice failed";
    return nullptr;
  }
  auto it = handles.find(dev);
  if (it != handles.end()) return it->second;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    *err = "the first dsa_indexer_project call on a thread and device creates a rocBLAS handle, which allocates: "
           "make one call outside graph capture first";
    *unsupported = true;
    return nullptr;
  }
  rocblas_handle h = nullptr;
  rocblas_status s = rocblas_create_handle(&h);
  if (s != rocblas_status_success) {
    *err = std::string("rocblas_create_handle: ") + blas_name(s);
    return nullptr;
  }
  // reproducible results: no split-K accumulation through atomics
  rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed);
  handles.emplace(dev, h);
  return h;
}

}  // namespace

int proj_block_tokens(int T, int requested) {
  const int blk = requested > 0 ? requested : 65536;
  return T < blk ? T : blk;
}

// Workspace: fp32 query staging for one token block, fp32 key/weight
// projections of all tokens, [W_IK; W_IW], rocBLAS scratch.
size_t proj_workspace_bytes(int T, int hidden, int block_tokens) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t blk = (size_t)proj_block_tokens(T, block_tokens);
  return up(blk * kQCols * 4) + up((size_t)T * kKWCols * 4) + up((size_t)kKWCols * hidden * 2) + kProjBlasScratch;
}

int run_projection(const ProjProblem& p, int out, uint8_t* q_out, float* q_scale, uint8_t* k_out, float* k_scale,
                   float* w_out, uint8_t* ws, hipStream_t st, std::string* err) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const int blk = proj_block_tokens(p.T, p.block_tokens);
  float* dq = reinterpret_cast<float*>(ws);
  float* dkw = reinterpret_cast<float*>(ws + up((size_t)blk * kQCols * 4));
  uint16_t* wcat = reinterpret_cast<uint16_t*>(ws + up((size_t)blk * kQCols * 4) + up((size_t)p.T * kKWCols * 4));
  uint8_t* scratch = reinterpret_cast<uint8_t*>(wcat) + up((size_t)kKWCols * p.hidden * 2);

  bool unsupported = false;
  rocblas_handle h = blas_handle(st, err, &unsupported);
  if (!h) return unsupported ? 2 : 1;
  rocblas_status s = rocblas_set_stream(h, st);
  if (s == rocblas_status_success) s = rocblas_set_workspace(h, scratch, kProjBlasScratch);
  if (s != rocblas_status_success) {
    *err = std::string("rocBLAS setup: ") + blas_name(s);
    return 1;
  }
  // [W_IK; W_IW] as one [192, hidden] operand, so X is read once
  const size_t wk_bytes = (size_t)128 * p.hidden * 2, ww_bytes = (size_t)64 * p.hidden * 2;
  if (hipMemcpyAsync(wcat, p.w_ik, wk_bytes, hipMemcpyDeviceToDevice, st) != hipSuccess ||
      hipMemcpyAsync(reinterpret_cast<uint8_t*>(wcat) + wk_bytes, p.w_iw, ww_bytes, hipMemcpyDeviceToDevice, st) !=
          hipSuccess) {
    *err = "hipMemcpyAsync of the key/weight projection matrices failed";
    return 1;
  }
  const float one = 1.0f, zero = 0.0f;
  // K^I and W^I of all tokens in one GEMM (a [T,192] fp32 result); the
  // thin product runs best over the whole token axis
  {
    const int slot = prof_open("gemm_kw_proj", st);
    s = rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, kKWCols, p.T, p.hidden, &one, wcat,
                        rocblas_datatype_bf16_r, p.hidden, p.x, rocblas_datatype_bf16_r, p.hidden, &zero, dkw,
                        rocblas_datatype_f32_r, kKWCols, dkw, rocblas_datatype_f32_r, kKWCols, rocblas_datatype_f32_r,
                        rocblas_gemm_algo_standard, 0, 0);
    prof_close(slot, st);
    if (s != rocblas_status_success) {
      *err = std::string("rocblas_gemm_ex (key/weight projection): ") + blas_name(s);
      return 1;
    }
  }
  for (int t0 = 0; t0 < p.T; t0 += blk) {
    const int n = p.T - t0 < blk ? p.T - t0 : blk;
    // column-major view: D^T[o, t] = sum_i W[o, i] * A[t, i]  (op(W) = W^T stored row-major [o, i])
    int slot = prof_open("gemm_q_proj", st);
    s = rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, kQCols, n, p.q_latent, &one, p.w_iq,
                        rocblas_datatype_bf16_r, p.q_latent, p.c_q + (size_t)t0 * p.q_latent, rocblas_datatype_bf16_r,
                        p.q_latent, &zero, dq, rocblas_datatype_f32_r, kQCols, dq, rocblas_datatype_f32_r, kQCols,
                        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    prof_close(slot, st);
    if (s != rocblas_status_success) {
      *err = std::string("rocblas_gemm_ex (query projection): ") + blas_name(s);
      return 1;
    }
    const size_t eq = out == 0 ? 1 : out == 1 ? 2 : 4;
    uint8_t* qo = q_out + (size_t)t0 * kQCols * eq;
    uint8_t* ko = k_out + (size_t)t0 * 128 * eq;
    float* qsc = q_scale ? q_scale + t0 : nullptr;
    float* ksc = k_scale ? k_scale + t0 : nullptr;
    float* wo = w_out + (size_t)t0 * 64;
    const float* kwb = dkw + (size_t)t0 * kKWCols;
    slot = prof_open("k_proj_out", st);
    if (out == 0)
      hipLaunchKernelGGL(k_proj_out<0>, dim3(n), dim3(kOutThreads), 0, st, dq, kwb, qo, qsc, ko, ksc, wo);
    else if (out == 1)
      hipLaunchKernelGGL(k_proj_out<1>, dim3(n), dim3(kOutThreads), 0, st, dq, kwb, qo, qsc, ko, ksc, wo);
    else
      hipLaunchKernelGGL(k_proj_out<2>, dim3(n), dim3(kOutThreads), 0, st, dq, kwb, qo, qsc, ko, ksc, wo);
    prof_close(slot, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      *err = std::string("HIP launch failed: ") + hipGetErrorString(e);
      return 1;
    }
  }
  return 0;
}

}  // namespace dsa
