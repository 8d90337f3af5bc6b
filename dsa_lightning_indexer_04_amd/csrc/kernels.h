// kernels.h -- host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct Problem {
  int B, Q, N, dtype;
  const uint8_t* q;
  const uint8_t* k;
  const float* w;
  const float* q_scale;
  const float* k_scale;
  const int32_t* pos;
};

// Full [B,Q,N] score matrix, -inf where not visible.
hipError_t launch_scores(const Problem& p, float* scores, hipStream_t st);

// Exact Top-K of every row of a [B*Q, N] score matrix (visibility from pos).
hipError_t launch_select_rows(const Problem& p, const float* scores, int topk, int32_t* out_idx,
                              float* out_score, hipStream_t st);

// Streaming Top-K: scores key tiles and keeps per-row candidate records in
// `cand` ([B*Q][cap] uint64), never storing the score matrix.
hipError_t launch_topk_stream(const Problem& p, int topk, int cap, uint64_t* cand, int32_t* out_idx,
                              float* out_score, hipStream_t st);

// Candidate capacity (records per row) used by the streaming Top-K.
inline int stream_capacity(int topk) { return 4 * topk + 128; }

}  // namespace dsa
