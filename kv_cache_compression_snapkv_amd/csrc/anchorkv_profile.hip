// Opt-in stage profiler: HIP events recorded between the stages of a call.
#include <hip/hip_runtime.h>

#include "anchorkv_internal.hpp"

namespace akv {

namespace {
constexpr int kMaxEvents = 1024;
struct Prof {
  int on = 0;
  int n = 0;
  bool created = false;
  hipEvent_t ev[kMaxEvents];
  const char* name[kMaxEvents];  // nullptr marks the start of a call
};
Prof g_prof;
}  // namespace

void prof_call_begin(void* stream) {
  if (!g_prof.on || g_prof.n >= kMaxEvents) return;
  if (hipEventRecord(g_prof.ev[g_prof.n], reinterpret_cast<hipStream_t>(stream)) == hipSuccess)
    g_prof.name[g_prof.n++] = nullptr;
}

void prof_mark(void* stream, const char* stage) {
  if (!g_prof.on || g_prof.n >= kMaxEvents) return;
  if (hipEventRecord(g_prof.ev[g_prof.n], reinterpret_cast<hipStream_t>(stream)) == hipSuccess)
    g_prof.name[g_prof.n++] = stage;
}

}  // namespace akv

using namespace akv;

extern "C" int anchorkv_profile_enable(int enable) {
  if (enable && !g_prof.created) {
    for (int i = 0; i < kMaxEvents; ++i)
      if (hipEventCreate(&g_prof.ev[i]) != hipSuccess) return fail(ANCHORKV_E_HIP, "anchorkv_profile_enable: hipEventCreate failed");
    g_prof.created = true;
  }
  g_prof.on = enable ? 1 : 0;
  g_prof.n = 0;
  return 0;
}

extern "C" int anchorkv_profile_read(const char** names, float* ms, int max_stages, int* n_stages) {
  if (!names || !ms || !n_stages || max_stages < 0) return fail(ANCHORKV_E_ARG, "anchorkv_profile_read: bad argument");
  *n_stages = 0;
  if (!g_prof.created || g_prof.n == 0) return 0;
  if (hipEventSynchronize(g_prof.ev[g_prof.n - 1]) != hipSuccess)
    return fail(ANCHORKV_E_HIP, "anchorkv_profile_read: hipEventSynchronize failed");
  int k = 0;
  for (int i = 1; i < g_prof.n && k < max_stages; ++i) {
    if (!g_prof.name[i]) continue;  // start of a new call
    float t = 0.0f;
    if (hipEventElapsedTime(&t, g_prof.ev[i - 1], g_prof.ev[i]) != hipSuccess)
      return fail(ANCHORKV_E_HIP, "anchorkv_profile_read: hipEventElapsedTime failed");
    names[k] = g_prof.name[i];
    ms[k] = t;
    ++k;
  }
  *n_stages = k;
  g_prof.n = 0;
  return 0;
}
