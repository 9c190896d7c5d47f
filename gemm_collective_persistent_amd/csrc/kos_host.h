// Host-side helpers shared by the entry points: error reporting, device
// properties, workspace and option checks.
#pragma once

#include <hip/hip_runtime.h>

#include "kos_common.h"

namespace kos {

// Records a thread-local message for kos_last_error() and returns `s`.
kos_status fail(kos_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

struct DeviceInfo {
  int device = -1;
  int cus = 0;
  bool gfx950 = false;
};

// Properties of the current device (cached per device).
kos_status current_device(DeviceInfo* out);

// Validates a workspace pointer/size.
kos_status check_workspace(const void* ws, size_t ws_bytes);

// Initial crew (workgroups that start in the communication role) of one op,
// per mode and peer link.  A property of the op and the link, set once and
// never per shape or call: there is no tuned split.
constexpr int kCrewHalfGrid = -2;   // a CrewDefaults value: half of the launch grid
struct CrewDefaults {
  int fused_hbm, fused_host;   // FUSED: the crew that starts communicating, then switches
  int fixed_hbm, fixed_host;   // FIXED: the crew that only communicates
};

// Fills `o` from `in` (NULL -> defaults), resolving the default crew size
// for the op, mode and peer link, and the grid.  Validates enums and ranges.
kos_status resolve_opts(const kos_opts* in, const DeviceInfo& dev, const CrewDefaults& crew, kos_opts* o);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch `l` of a traced call records into its own slot of the trace
// region (null when tracing is off).
inline kos_trace_rec* trace_slot(void* ws, int traced, int l) {
  return traced ? reinterpret_cast<kos_trace_rec*>(static_cast<char*>(ws) + kTraceOffset) + (size_t)l * kTraceSlotRecords
                : nullptr;
}

// Maps a launch error to a status.
kos_status launch_status(const char* what);

}  // namespace kos
