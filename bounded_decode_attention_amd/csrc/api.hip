// Host-side helpers shared by all entry points: status strings, device check,
// cache descriptor validation.
#include <string.h>

#include <vector>

#include "common.h"

namespace kvb {

namespace {
struct TraceState {
  int mask = 0;
  int used = 0;
  std::vector<hipEvent_t> start, stop;
  std::vector<int> kernel;
};
TraceState g_trace;
}  // namespace

TraceScope::TraceScope(int k, hipStream_t s) : slot(-1), stream(s) {
  if (!(g_trace.mask & k) || g_trace.used >= (int)g_trace.start.size()) return;
  slot = g_trace.used++;
  g_trace.kernel[slot] = k;
  hipEventRecord(g_trace.start[slot], s);
}

TraceScope::~TraceScope() {
  if (slot >= 0) hipEventRecord(g_trace.stop[slot], stream);
}

int32_t check_device() {
  static int cached[64];  // 0 unknown, 1 ok, -1 not gfx950
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KVB_EDEVICE;
  if (dev < 64 && cached[dev]) return cached[dev] > 0 ? KVB_OK : KVB_EDEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KVB_EDEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cached[dev] = ok ? 1 : -1;
  return ok ? KVB_OK : KVB_EDEVICE;
}

bool cache_dims_ok(const kvb_cache* c) {
  return c && c->B >= 1 && c->Hkv >= 1 && c->cap >= 1 && c->cap < (1 << 30) && c->D >= 1 &&
         c->D <= 256 && (long long)c->B * c->Hkv <= (1 << 20);
}

int32_t check_cache(const kvb_cache* c, bool need_kv) {
  if (!c) return KVB_EINVAL;
  if (c->B < 1 || c->Hkv < 1 || c->cap < 1 || c->cap >= (1 << 30) || c->D < 1) return KVB_EINVAL;
  if (!c->pos || !c->len) return KVB_EINVAL;
  if (need_kv && (!c->k || !c->v)) return KVB_EINVAL;
  // rows, positions and log betas are read 16 bytes at a time
  auto mis = [](const void* p) { return ((uintptr_t)p & 15u) != 0; };
  if (mis(c->k) || mis(c->v) || mis(c->pos) || mis(c->log_beta)) return KVB_EINVAL;
  if (c->dtype != KVB_F32 && c->dtype != KVB_BF16) return KVB_EUNSUPPORTED;
  if (c->D % 8 != 0 || c->D > 256) return KVB_EUNSUPPORTED;
  if (c->dtype == KVB_BF16 && c->D != 64 && c->D != 128) return KVB_EUNSUPPORTED;
  if ((long long)c->B * c->Hkv > (1 << 20)) return KVB_EINVAL;
  return KVB_OK;
}

}  // namespace kvb

using namespace kvb;

extern "C" void kvb_trace_disable(void) {
  for (size_t i = 0; i < g_trace.start.size(); ++i) {
    hipEventDestroy(g_trace.start[i]);
    hipEventDestroy(g_trace.stop[i]);
  }
  g_trace = TraceState();
}

extern "C" int32_t kvb_trace_enable(int32_t capacity, int32_t kernel_mask) {
  kvb_trace_disable();
  if (capacity < 0 || capacity > (1 << 20)) return KVB_EINVAL;
  if (capacity == 0 || kernel_mask == 0) return KVB_OK;
  int32_t st = check_device();
  if (st) return st;
  g_trace.start.resize(capacity);
  g_trace.stop.resize(capacity);
  g_trace.kernel.assign(capacity, 0);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&g_trace.start[i]) != hipSuccess ||
        hipEventCreate(&g_trace.stop[i]) != hipSuccess) {
      g_trace.start.resize(i);
      g_trace.stop.resize(i);
      kvb_trace_disable();
      return KVB_EDEVICE;
    }
  }
  g_trace.mask = kernel_mask;
  return KVB_OK;
}

extern "C" int32_t kvb_trace_read(int32_t* kernel_ids, float* ms, int32_t max) {
  const int n = g_trace.used < max ? g_trace.used : max;
  for (int i = 0; i < n; ++i) {
    float e = -1.f;
    if (hipEventSynchronize(g_trace.stop[i]) == hipSuccess)
      hipEventElapsedTime(&e, g_trace.start[i], g_trace.stop[i]);
    if (kernel_ids) kernel_ids[i] = g_trace.kernel[i];
    if (ms) ms[i] = e;
  }
  return n;
}

extern "C" void kvb_trace_reset(void) { g_trace.used = 0; }

extern "C" const char* kvb_strerror(int32_t status) {
  switch (status) {
    case KVB_OK: return "ok";
    case KVB_EINVAL: return "invalid argument";
    case KVB_EUNSUPPORTED: return "unsupported dtype/head_dim/group size";
    case KVB_ECAPACITY: return "cache capacity exceeded";
    case KVB_EWORKSPACE: return "workspace missing or too small";
    case KVB_EDEVICE: return "no gfx950 device";
    case KVB_ELAUNCH: return "kernel launch failed";
    case KVB_ERANGE: return "input value outside the supported range (saturated)";
    default: return "unknown status";
  }
}
