// Host-side helpers shared by all entry points: status strings, device check,
// cache descriptor validation.
#include <string.h>

#include "common.h"

namespace kvb {

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

int32_t check_cache(const kvb_cache* c, bool need_kv) {
  if (!c) return KVB_EINVAL;
  if (c->B < 1 || c->Hkv < 1 || c->cap < 1 || c->cap >= (1 << 30) || c->D < 1) return KVB_EINVAL;
  if (!c->pos || !c->len) return KVB_EINVAL;
  if (need_kv && (!c->k || !c->v)) return KVB_EINVAL;
  if (c->dtype != KVB_F32 && c->dtype != KVB_BF16) return KVB_EUNSUPPORTED;
  if (c->D % 8 != 0 || c->D > 256) return KVB_EUNSUPPORTED;
  if (c->dtype == KVB_BF16 && c->D != 64 && c->D != 128) return KVB_EUNSUPPORTED;
  if ((long long)c->B * c->Hkv > (1 << 20)) return KVB_EINVAL;
  return KVB_OK;
}

}  // namespace kvb

extern "C" const char* kvb_strerror(int32_t status) {
  switch (status) {
    case KVB_OK: return "ok";
    case KVB_EINVAL: return "invalid argument";
    case KVB_EUNSUPPORTED: return "unsupported dtype/head_dim/group size";
    case KVB_ECAPACITY: return "cache capacity exceeded";
    case KVB_EWORKSPACE: return "workspace missing or too small";
    case KVB_EDEVICE: return "no gfx950 device";
    case KVB_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
