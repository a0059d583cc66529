// fa_api.hip — status strings and the kernel-timing hooks of libfa.so.
#include <vector>

#include "fa_host.h"

namespace fa {

namespace {
struct Profiler {
  bool on = false;
  int capacity = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;   // 2 per slot
  std::vector<int> kind;        // kernel kind per slot
  int open_slot = -1;
};
Profiler g_prof;

void prof_destroy() {
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.kind.clear();
  g_prof.capacity = g_prof.used = 0;
  g_prof.open_slot = -1;
}
}  // namespace

void prof_before(int kind, hipStream_t s) {
  if (!g_prof.on || g_prof.used >= g_prof.capacity) {
    g_prof.open_slot = -1;
    return;
  }
  const int slot = g_prof.used++;
  g_prof.kind[slot] = kind;
  g_prof.open_slot = slot;
  (void)hipEventRecord(g_prof.ev[2 * slot], s);
}

void prof_after(int kind, hipStream_t s) {
  (void)kind;
  if (g_prof.open_slot < 0) return;
  (void)hipEventRecord(g_prof.ev[2 * g_prof.open_slot + 1], s);
  g_prof.open_slot = -1;
}

}  // namespace fa

using namespace fa;

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCRATCH_LIMIT: return "request exceeds the static scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

extern "C" const char* fa_kernel_name(int kind) {
  switch (kind) {
    case FA_KERNEL_FWD: return "fwd";
    case FA_KERNEL_BWD_PREPROCESS: return "bwd_preprocess";
    case FA_KERNEL_BWD_DKDV: return "bwd_dkdv";
    case FA_KERNEL_BWD_DQ: return "bwd_dq";
    case FA_KERNEL_DECODE_SPLIT: return "decode_split";
    case FA_KERNEL_DECODE_COMBINE: return "decode_combine";
    default: return "unknown";
  }
}

extern "C" int fa_profiler_enable(int enable, int capacity) {
  prof_destroy();
  g_prof.on = false;
  if (!enable) return FA_OK;
  if (capacity < 1) return FA_ERR_INVALID_ARG;
  g_prof.ev.resize(2 * (size_t)capacity);
  g_prof.kind.assign(capacity, 0);
  // timing-only events: without the system-scope release fence a record
  // would otherwise add (writing back the kernel's dirty lines), the pair
  // brackets the kernel's own execution
  for (size_t i = 0; i < g_prof.ev.size(); ++i) {
    if (hipEventCreateWithFlags(&g_prof.ev[i], hipEventDisableSystemFence) != hipSuccess) {
      g_prof.ev.resize(i);
      prof_destroy();
      return FA_ERR_LAUNCH;
    }
  }
  g_prof.capacity = capacity;
  g_prof.on = true;
  return FA_OK;
}

extern "C" int fa_profiler_reset(void) {
  g_prof.used = 0;
  g_prof.open_slot = -1;
  return FA_OK;
}

extern "C" int fa_profiler_read(int kind, double* total_ms, long* launches) {
  if (kind < 0 || kind >= FA_KERNEL_KIND_COUNT || !total_ms || !launches) return FA_ERR_INVALID_ARG;
  double tot = 0.0;
  long n = 0;
  for (int s = 0; s < g_prof.used; ++s) {
    if (g_prof.kind[s] != kind) continue;
    if (hipEventSynchronize(g_prof.ev[2 * s + 1]) != hipSuccess) return FA_ERR_LAUNCH;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, g_prof.ev[2 * s], g_prof.ev[2 * s + 1]) != hipSuccess) return FA_ERR_LAUNCH;
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return FA_OK;
}
