// profile.cpp -- optional per-kernel HIP-event timing (dsa_indexer_profile.h).
#include <hip/hip_runtime_api.h>

#include <cstring>
#include <vector>

#include "../../include/dsa_indexer_profile.h"
#include "kernels.h"

namespace dsa {
namespace {
struct Rec {
  const char* name;
  hipEvent_t a, b;
};
bool g_on = false;
std::vector<Rec> g_recs;
}  // namespace

int prof_open(const char* name, hipStream_t st) {
  if (!g_on) return -1;
  Rec r{name, nullptr, nullptr};
  if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return -1;
  hipEventRecord(r.a, st);
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

void prof_close(int slot, hipStream_t st) {
  if (slot >= 0 && slot < (int)g_recs.size()) hipEventRecord(g_recs[slot].b, st);
}
}  // namespace dsa

extern "C" {

int dsa_indexer_profile_begin(void) {
  for (auto& r : dsa::g_recs) {
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  dsa::g_recs.clear();
  dsa::g_on = true;
  return 0;
}

int dsa_indexer_profile_end(const char** names, int32_t* launches, double* mean_ms, int max_kernels) {
  dsa::g_on = false;
  std::vector<const char*> nm;
  std::vector<double> tot;
  std::vector<int> cnt;
  int rc = 0;
  for (auto& r : dsa::g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) rc = -1;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) rc = -1;
    size_t i = 0;
    while (i < nm.size() && std::strcmp(nm[i], r.name) != 0) ++i;
    if (i == nm.size()) {
      nm.push_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[i] += ms;
    cnt[i] += 1;
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  dsa::g_recs.clear();
  if (rc) return -1;
  for (size_t i = 0; i < nm.size() && (int)i < max_kernels; ++i) {
    if (names) names[i] = nm[i];
    if (launches) launches[i] = cnt[i];
    if (mean_ms) mean_ms[i] = tot[i] / cnt[i];
  }
  return (int)nm.size();
}

}  // extern "C"
