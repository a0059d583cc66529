// fa_host.h — host-side helpers shared by the entry points: argument checks,
// launch-grid remapping for the 8 XCDs, and the kernel-timing hooks.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

inline bool aligned16(const void* p) { return p && (((uintptr_t)p) & 15u) == 0; }
inline bool opt_aligned16(const void* p) { return p == nullptr || aligned16(p); }
inline bool aligned4(const void* p) { return p && (((uintptr_t)p) & 3u) == 0; }

// Checks shared by the dense and packed entry points.
inline int check_common(int Hq, int Hkv, int D, int dtype, float scale, int wl, int wr,
                        float softcap) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
  if (D < 1) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (wl < -1 || wr < -1) return FA_ERR_INVALID_ARG;
  if (!(softcap >= 0.0f) || !isfinite(softcap)) return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Work-group ids are handed to the 8 XCDs round-robin (id % 8).  The kernels
// remap the hardware id so that each XCD receives one contiguous block of
// logical tiles, which keeps tiles that share K/V rows on the same L2.
__device__ __forceinline__ int xcd_remap(int hw_id, int n) {
  const int per = n / 8;
  if (hw_id >= per * 8) return hw_id;
  return (hw_id & 7) * per + (hw_id >> 3);
}

// ---- kernel timing (implemented in fa_api.hip) ----
void prof_before(int kind, hipStream_t s);
void prof_after(int kind, hipStream_t s);

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
