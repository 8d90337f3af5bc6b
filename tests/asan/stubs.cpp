// Host-only stand-ins for the kernel launchers and the HIP calls that the C
// ABI (abi.cpp) makes, so that its argument checks and workspace carving can
// run under AddressSanitizer on a machine without a GPU.  Each launcher
// records that it was called and reports success; nothing touches device
// memory.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <string>

#include "../../dsa_lightning_indexer_04_amd/csrc/kernels.h"

int g_launches = 0;

namespace dsa {
int prof_open(const char*, hipStream_t) { return -1; }
void prof_close(int, hipStream_t) {}
hipError_t launch_scores(const Problem&, float*, uint32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_select_rows(const Problem&, const float*, const uint32_t*, int, int32_t*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_topk_stream(const Problem&, int, int, uint64_t*, int32_t*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_topk_stream_rows(const Problem&, int, int, uint64_t*, int32_t*, float*, const int32_t*, const char*,
                                   hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_seed_prep(const Problem&, int, const int32_t*, int32_t*, int32_t*, uint32_t*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_key_norms(const Problem&, float*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_anchor_rows(const Problem&, int, int32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_anchor_seeds(const Problem&, int, int, const int32_t*, int, int32_t*, int32_t*, uint32_t*, int32_t*,
                               hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_seed_pack(const Problem&, const int32_t*, const int32_t*, int, uint8_t*, float*, int32_t*,
                            hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_plan(const Problem&, int, const int32_t*, const int32_t*, int, const int32_t*, const uint8_t*,
                       uint8_t*, float*, float*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_topk_pruned(const Problem&, int, int, uint64_t*, int32_t*, float*, const PrunedBuffers&,
                              hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int prune_mask_words(int N, int row_bytes) { return (std::min(N, kPruneChunkBytes / row_bytes) + 127) / 128 * 2; }
int proj_block_tokens(int T, int requested) { return std::min(T, requested > 0 ? requested : 65536); }
size_t proj_workspace_bytes(int T, int hidden, int block_tokens) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up((size_t)proj_block_tokens(T, block_tokens) * 8192 * 4) + up((size_t)T * 192 * 4) +
         up((size_t)192 * hidden * 2) + kProjBlasScratch;
}
int run_projection(const ProjProblem&, int, uint8_t*, float*, uint8_t*, float*, float*, uint8_t*, hipStream_t,
                   std::string*) {
  ++g_launches;
  return 0;
}
int mla_splits(int rows, int requested) {
  if (requested > 0) return std::min(requested, 8);
  return rows < 256 ? std::min(8, (512 + rows - 1) / rows) : 1;
}
hipError_t launch_sparse_mla(const MlaProblem&, float, uint16_t*, float*, float*, int32_t*, int, float*, float*,
                             hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int mfma_ceiling_workgroups() { return 512; }
hipError_t launch_mfma_ceiling(int, int, int, int, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int noalloc_scratch(void** ptr, std::string*) {
  static char fake[256] __attribute__((aligned(256)));
  *ptr = fake;  // never dereferenced: the launchers above are stand-ins
  return 0;
}
}  // namespace dsa

extern "C" {
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t hipMemcpy2DAsync(void*, size_t, const void*, size_t, size_t, size_t, hipMemcpyKind, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}
