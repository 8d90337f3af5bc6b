// Drives every C ABI entry point through its argument checks and its
// success paths (with the launchers stubbed out), for a build under
// AddressSanitizer / UndefinedBehaviorSanitizer.  Pointers are fake device
// addresses: the ABI only compares and offsets them.  Exit status 0 iff
// every return code is the expected one.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "dsa_indexer.h"
#include "dsa_indexer_profile.h"

extern int g_launches;
static int g_checks = 0, g_bad = 0;

#define EXPECT(expr, code)                                                                  \
  do {                                                                                      \
    const int rc_ = (expr);                                                                 \
    ++g_checks;                                                                             \
    if (rc_ != (code)) {                                                                    \
      ++g_bad;                                                                              \
      std::printf("line %d: %s returned %d, expected %d (%s)\n", __LINE__, #expr, rc_, (code), \
                  dsa_indexer_last_error());                                               \
    }                                                                                       \
  } while (0)

static void* P(uint64_t mib) { return reinterpret_cast<void*>(uintptr_t(mib) << 20); }

static dsa_indexer_inputs inputs(int B, int Q, int N, int dtype) {
  dsa_indexer_inputs in;
  std::memset(&in, 0, sizeof(in));
  in.batch = B, in.num_q = Q, in.num_k = N, in.heads = 64, in.head_dim = 128, in.dtype = dtype;
  in.q = P(1 << 10), in.k = P(2 << 10), in.w = static_cast<const float*>(P(3 << 10));
  in.positions = static_cast<const int32_t*>(P(4 << 10));
  if (dtype == DSA_FP8_E4M3) in.q_scale = static_cast<const float*>(P(5 << 10)), in.k_scale = static_cast<const float*>(P(6 << 10));
  return in;
}

int main() {
  int32_t* oi = static_cast<int32_t*>(P(10 << 10));
  float* os = static_cast<float*>(P(11 << 10));
  void* ws = P(12 << 10);
  for (int dt : {DSA_BF16, DSA_FP8_E4M3}) {
    for (int shape = 0; shape < 3; ++shape) {
      const int B = shape == 2 ? 64 : 1, Q = shape == 0 ? 7 : shape == 1 ? 8192 : 1, N = shape == 0 ? 300 : 131072;
      dsa_indexer_inputs in = inputs(B, Q, N, dt);
      for (uint32_t flags : {0u, (uint32_t)DSA_FLAG_ROUTE_STREAM, (uint32_t)DSA_FLAG_ROUTE_SPLIT}) {
        in.flags = flags;
        const size_t need = dsa_indexer_workspace_bytes(DSA_OP_TOPK, &in, 2048, nullptr);
        EXPECT(need > 0 ? 0 : 1, 0);
        EXPECT(dsa_indexer_topk(&in, 2048, oi, os, ws, need, nullptr), DSA_OK);
        EXPECT(dsa_indexer_topk(&in, 2048, oi, os, ws, need - 1, nullptr), DSA_ERR_WORKSPACE);
        EXPECT(dsa_indexer_topk(&in, 2048, oi, os, static_cast<char*>(ws) + 16, need, nullptr),
               DSA_ERR_INVALID_ARG);  // workspace not 256-byte aligned
        EXPECT(dsa_indexer_topk(&in, 0, oi, os, ws, need, nullptr), DSA_ERR_INVALID_ARG);
        EXPECT(dsa_indexer_topk(&in, 4097, oi, os, ws, need, nullptr), DSA_ERR_UNSUPPORTED);
        EXPECT(dsa_indexer_topk(&in, 2048, static_cast<int32_t*>(P(1 << 10)), os, ws, need, nullptr),
               DSA_ERR_INVALID_ARG);  // out_idx over q
        const int want = need <= DSA_NOALLOC_SCRATCH_BYTES ? DSA_OK : DSA_ERR_WORKSPACE;
        EXPECT(dsa_indexer_topk_noalloc(&in, 2048, oi, os, nullptr), want);
      }
      in.flags = 3;
      EXPECT(dsa_indexer_topk(&in, 16, oi, os, ws, 1 << 30, nullptr), DSA_ERR_INVALID_ARG);
      in.flags = 0;
      EXPECT(dsa_indexer_scores(&in, static_cast<float*>(P(20 << 10)), nullptr), DSA_OK);
      dsa_prune_opts po;
      std::memset(&po, 0, sizeof(po));
      const size_t pneed = dsa_indexer_workspace_bytes(DSA_OP_TOPK_PRUNED, &in, 2048, &po);
      EXPECT(pneed > 0 ? 0 : 1, 0);
      dsa_prune_stats st;
      std::memset(&st, 0, sizeof(st));
      st.tau = static_cast<float*>(P(30 << 10));
      st.plan_rows = P(31 << 10);
      st.plan_coef = static_cast<float*>(P(40 << 10));
      st.plan_misc = static_cast<float*>(P(41 << 10));
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, &st, ws, pneed, nullptr), DSA_OK);
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, &st, ws, pneed - 8, nullptr), DSA_ERR_WORKSPACE);
      po.num_retained = 31;
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, nullptr, ws, pneed, nullptr), DSA_ERR_UNSUPPORTED);
      po.num_retained = 0;
      po.flags = DSA_PRUNE_START_AT_TAU;
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, &st, ws, pneed, nullptr), DSA_OK);
      po.flags = DSA_PRUNE_START_AT_TAU | DSA_PRUNE_COMPACT_RECORDS;
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, &st, ws, pneed, nullptr), DSA_OK);
      po.flags = DSA_PRUNE_ANCHOR_SEEDS;  // 12288 seeds: 6 anchor rows of top-2048
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, &st, ws, pneed, nullptr), DSA_OK);
      po.num_seeds = 1024;  // fewer seeds than topk
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, &st, ws, pneed, nullptr), DSA_ERR_INVALID_ARG);
      po.num_seeds = 0;
      po.flags = 8;
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, &st, ws, pneed, nullptr), DSA_ERR_INVALID_ARG);
      EXPECT(dsa_indexer_workspace_bytes(DSA_OP_TOPK_PRUNED, &in, 2048, &po) == 0 ? 0 : 1, 0);
      po.flags = 0;
      st.tau = static_cast<float*>(ws);  // stats inside the workspace
      EXPECT(dsa_indexer_topk_pruned(&in, 2048, &po, oi, os, &st, ws, pneed, nullptr), DSA_ERR_INVALID_ARG);
    }
    dsa_indexer_inputs bad = inputs(1, 4, 64, dt);
    bad.heads = 32;
    EXPECT(dsa_indexer_topk(&bad, 16, oi, os, ws, 1 << 30, nullptr), DSA_ERR_UNSUPPORTED);
    bad = inputs(1, 4, 64, dt);
    bad.q = static_cast<const char*>(P(1 << 10)) + 4;  // misaligned
    EXPECT(dsa_indexer_topk(&bad, 16, oi, os, ws, 1 << 30, nullptr), DSA_ERR_INVALID_ARG);
    EXPECT(dsa_indexer_topk(nullptr, 16, oi, os, ws, 1 << 30, nullptr), DSA_ERR_INVALID_ARG);
  }
  // projections
  dsa_proj_inputs pi;
  std::memset(&pi, 0, sizeof(pi));
  pi.num_tokens = 5000, pi.hidden = 7168, pi.q_latent = 1536, pi.heads = 64, pi.head_dim = 128;
  pi.c_q = P(1 << 10), pi.x = P(2 << 10), pi.w_iq = P(3 << 10), pi.w_ik = P(4 << 10), pi.w_iw = P(5 << 10);
  for (int blk : {0, 64, 1000}) {
    pi.block_tokens = blk;
    const size_t need = dsa_indexer_project_workspace_bytes(&pi);
    EXPECT(need > 0 ? 0 : 1, 0);
    EXPECT(dsa_indexer_project(&pi, DSA_FP8_E4M3, P(10 << 10), static_cast<float*>(P(11 << 10)), P(12 << 10),
                               static_cast<float*>(P(13 << 10)), static_cast<float*>(P(14 << 10)), P(16 << 10), need,
                               nullptr),
           DSA_OK);
    EXPECT(dsa_indexer_project(&pi, 9, P(10 << 10), nullptr, P(12 << 10), nullptr, static_cast<float*>(P(14 << 10)),
                               P(16 << 10), need, nullptr),
           DSA_ERR_UNSUPPORTED);
  }
  pi.block_tokens = 7;
  EXPECT(dsa_indexer_project_workspace_bytes(&pi) == 0 ? 0 : 1, 0);
  // sparse MLA
  dsa_mla_inputs mi;
  std::memset(&mi, 0, sizeof(mi));
  mi.batch = 1, mi.num_q = 8, mi.num_k = 4096, mi.heads = 128, mi.latent_dim = 512, mi.rope_dim = 64, mi.topk = 2048;
  mi.q = P(1 << 10), mi.kv = P(2 << 10), mi.indices = static_cast<const int32_t*>(P(3 << 10));
  for (int sp : {0, 1, 8}) {
    mi.num_splits = sp;
    const size_t need = dsa_sparse_mla_workspace_bytes(&mi);
    EXPECT(need > 0 ? 0 : 1, 0);
    EXPECT(dsa_sparse_mla(&mi, 0.04f, P(10 << 10), static_cast<float*>(P(11 << 10)), P(12 << 10), need, nullptr),
           DSA_OK);
    EXPECT(dsa_sparse_mla(&mi, -1.0f, P(10 << 10), nullptr, P(12 << 10), need, nullptr), DSA_ERR_INVALID_ARG);
  }
  mi.num_splits = 9;
  EXPECT(dsa_sparse_mla_workspace_bytes(&mi) == 0 ? 0 : 1, 0);
  // sustained-rate probe: the count alone, a launch, a short buffer
  int32_t wg = 0;
  EXPECT(dsa_indexer_mfma_ceiling(DSA_BF16, 1, 64, nullptr, 0, nullptr, &wg), DSA_OK);
  EXPECT(wg > 0 ? 0 : 1, 0);
  EXPECT(dsa_indexer_mfma_ceiling(DSA_FP8_E4M3, 0, 64, static_cast<float*>(P(20 << 10)), (size_t)wg * 256, nullptr, &wg),
         DSA_OK);
  EXPECT(dsa_indexer_mfma_ceiling(DSA_BF16, 0, 64, static_cast<float*>(P(20 << 10)), (size_t)wg * 256 - 1, nullptr, &wg),
         DSA_ERR_INVALID_ARG);
  std::printf("%d checks, %d failed, %d stubbed launches\n", g_checks, g_bad, g_launches);
  return g_bad ? 1 : 0;
}
