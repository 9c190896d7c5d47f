// Layout of the workspace shared by host and device code.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/kos.h"

namespace kos {

constexpr int kNumHeads = 8;

// First 256 bytes of the workspace.  All zero between calls except `status`.
struct WsHeader {
  uint32_t ticket;          // arrival counter: role assignment
  uint32_t exit_count;      // departure counter: last one out resets
  uint32_t head[kNumHeads]; // queue heads
  uint32_t status;          // first device-side error (sticky)
  uint32_t err_info;        // which entry raised it
  uint32_t abort;           // non-zero: drain and exit
  uint32_t pad[64 - 13];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

constexpr size_t kCountersOffset = 4096;                 // ready counters
constexpr size_t kMaxCounters = (size_t(1) << 20) / 4;   // 1 MiB of uint32
constexpr size_t kScratchOffset = kCountersOffset + (size_t(1) << 20);
constexpr size_t kScratchBytes = size_t(15) << 20;       // per-op scratch
constexpr size_t kTraceOffset = kScratchOffset + kScratchBytes;      // timelines (kos_opts.trace)
// one slot of KOS_TRACE_MAX_WG rows per launch of a call (the unfused
// baselines launch up to KOS_TRACE_LAUNCHES kernels per call)
constexpr size_t kTraceSlotRecords = (size_t)KOS_TRACE_MAX_WG * KOS_TRACE_RECORDS;
constexpr size_t kTraceBytes = KOS_TRACE_LAUNCHES * kTraceSlotRecords * sizeof(kos_trace_rec);
constexpr size_t kWorkspaceBytes = kTraceOffset + kTraceBytes;       // 24 MiB + 4 KiB

constexpr uint32_t kDefaultSpinLimit = 1u << 24;  // x s_sleep(2) ~ a few seconds

}  // namespace kos
