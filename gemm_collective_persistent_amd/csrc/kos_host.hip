// Host-side common code of the C ABI: errors, device cache, workspace.
#include "kos_host.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

namespace kos {

namespace {
thread_local char g_msg[512] = "";

std::mutex g_dev_mu;
DeviceInfo g_dev[64];
}  // namespace

kos_status fail(kos_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

kos_status current_device(DeviceInfo* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(KOS_ERR_UNSUPPORTED, "no HIP device");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (d.device != dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(KOS_ERR_HIP, "hipGetDeviceProperties failed");
    d.cus = prop.multiProcessorCount;
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.device = dev;
  }
  *out = d;
  if (!d.gfx950) return fail(KOS_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return KOS_OK;
}

kos_status check_workspace(const void* ws, size_t ws_bytes) {
  if (!ws) return fail(KOS_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < kWorkspaceBytes)
    return fail(KOS_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, kWorkspaceBytes);
  if (!aligned16(ws)) return fail(KOS_ERR_ALIGN, "workspace not 16-byte aligned");
  return KOS_OK;
}

kos_status resolve_opts(const kos_opts* in, const DeviceInfo& dev, const CrewDefaults& crew, kos_opts* o) {
  kos_opts_default(o);
  if (in) *o = *in;
  if (o->mode < KOS_MODE_FUSED || o->mode > KOS_MODE_UNFUSED) return fail(KOS_ERR_ARG, "bad mode %d", o->mode);
  if (o->rs_order != KOS_RS_BAND && o->rs_order != KOS_RS_ROW) return fail(KOS_ERR_ARG, "bad rs_order %d", o->rs_order);
  if (o->peer_link != 0 && o->peer_link != 1) return fail(KOS_ERR_ARG, "bad peer_link %d", o->peer_link);
  if (o->policy != KOS_POLICY_DEFAULT && o->policy != KOS_POLICY_SWAPPED)
    return fail(KOS_ERR_ARG, "bad policy %d", o->policy);
  if (o->trace && o->grid > KOS_TRACE_MAX_WG)
    return fail(KOS_ERR_ARG, "tracing holds at most %d workgroups", KOS_TRACE_MAX_WG);
  if (o->grid == 0) o->grid = dev.cus;
  if (o->grid < 2 || o->grid > dev.cus)
    return fail(KOS_ERR_ARG, "grid %d outside [2, %d] (all workgroups must be co-resident)", o->grid, dev.cus);
  if (o->n_movers < 0) {
    const bool host = o->peer_link == 1;
    int c = o->mode == KOS_MODE_FIXED ? (host ? crew.fixed_host : crew.fixed_hbm)
                                      : (host ? crew.fused_host : crew.fused_hbm);
    if (c == kCrewHalfGrid) c = o->grid / 2;
    o->n_movers = c < o->grid ? c : o->grid - 1;   // a default never takes the whole grid
  }
  if (o->spin_limit == 0) o->spin_limit = kDefaultSpinLimit;
  return KOS_OK;
}

kos_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KOS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KOS_OK;
}

}  // namespace kos

using namespace kos;

extern "C" {

void kos_opts_default(kos_opts* o) {
  if (!o) return;
  memset(o, 0, sizeof(*o));
  o->mode = KOS_MODE_FUSED;
  o->n_movers = -1;
  o->rs_order = KOS_RS_BAND;
  o->grid = 0;
  o->spin_limit = 0;
  o->peer_link = 0;
}

size_t kos_workspace_bytes(void) { return kWorkspaceBytes; }

kos_status kos_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  kos_status st = check_workspace(ws, ws_bytes);
  if (st != KOS_OK) return st;
  if (hipMemsetAsync(ws, 0, kWorkspaceBytes, static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(KOS_ERR_HIP, "hipMemsetAsync of the workspace failed");
  return KOS_OK;
}

kos_status kos_workspace_status(void* ws, void* stream, kos_device_error* out) {
  if (out) {
    out->status = KOS_OK;
    out->entry = 0;
  }
  if (!ws) return fail(KOS_ERR_WORKSPACE, "workspace is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return fail(KOS_ERR_HIP, "stream synchronization failed");
  WsHeader h;
  if (hipMemcpy(&h, ws, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(KOS_ERR_HIP, "reading the workspace status failed");
  if (h.status == 0) return KOS_OK;
  const uint32_t zero = 0;
  if (hipMemcpy(reinterpret_cast<char*>(ws) + offsetof(WsHeader, status), &zero, 4, hipMemcpyHostToDevice) !=
      hipSuccess)
    return fail(KOS_ERR_HIP, "clearing the workspace status failed");
  if (out) {
    out->status = (int32_t)h.status;
    out->entry = h.err_info;
  }
  return fail(static_cast<kos_status>(h.status), "device error %u (entry %u)", h.status, h.err_info);
}

kos_status kos_workspace_trace(void* ws, kos_trace_rec* out, size_t n_records, void* stream) {
  if (!ws || (!out && n_records)) return fail(KOS_ERR_ARG, "null buffer");
  if (n_records > (size_t)KOS_TRACE_LAUNCHES * kTraceSlotRecords)
    return fail(KOS_ERR_ARG, "%zu records requested, the trace region holds %zu", n_records,
                (size_t)KOS_TRACE_LAUNCHES * kTraceSlotRecords);
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(KOS_ERR_HIP, "stream synchronization failed");
  if (n_records && hipMemcpy(out, static_cast<char*>(ws) + kTraceOffset, n_records * sizeof(kos_trace_rec),
                             hipMemcpyDeviceToHost) != hipSuccess)
    return fail(KOS_ERR_HIP, "reading the trace region failed");
  return KOS_OK;
}

const char* kos_last_error(void) { return g_msg; }

int32_t kos_device_cu_count(void) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // extern "C"
