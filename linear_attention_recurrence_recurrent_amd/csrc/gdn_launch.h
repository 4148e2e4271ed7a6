// Host-side helpers shared by the launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdn {

// GDN_OK, or GDN_EDEVICE with the HIP error text as the thread's last error.
inline int device_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return GDN_OK;
  char msg[200];
  std::snprintf(msg, sizeof(msg), "%s: %s", what, hipGetErrorString(e));
  set_error(msg);
  return GDN_EDEVICE;
}

// Whether `blocks` workgroups of `threads` fit one dispatch (kMaxLaunchItems
// work-items at most); otherwise sets the reason.  The descriptor check has
// already bounded every launch of a call (max_launch_items); this keeps a
// launcher from wrapping the grid if a shape ever escapes it.
inline bool launch_fits(int64_t blocks, int64_t threads, const char* what) {
  if (blocks > 0 && blocks <= kMaxLaunchItems / threads) return true;
  char msg[200];
  std::snprintf(msg, sizeof(msg), "%s: %lld workgroups of %lld threads do not fit one launch", what,
                (long long)blocks, (long long)threads);
  set_error(msg);
  return false;
}

// Scale folded into q-hat: 1/sqrt(Dk) when GDN_FOLD_Q_SCALE is set.
inline float q_scale(const gdn_desc& d) {
  return (d.flags & GDN_FOLD_Q_SCALE) ? 1.0f / std::sqrt((float)d.Dk) : 1.0f;
}

}  // namespace gdn
