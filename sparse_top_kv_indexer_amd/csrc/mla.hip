// Shared-latent (MLA-style) sparse attention on matrix cores.
#include "skv_device.h"

namespace skv {

bool mla_supported(const KvArgs& kv, int G) {
  (void)kv;
  (void)G;
  return false;
}

size_t mla_workspace_bytes(const KvArgs& kv, int G, int k) {
  (void)kv;
  (void)G;
  (void)k;
  return 0;
}

hipError_t launch_mla_attend(const KvArgs& kv, const void* q, int G, const int32_t* idx, int k,
                             const int32_t* lo, const int32_t* hi, float scale, float* out,
                             void* ws, size_t ws_bytes, hipStream_t s) {
  (void)kv; (void)q; (void)G; (void)idx; (void)k; (void)lo; (void)hi; (void)scale; (void)out;
  (void)ws; (void)ws_bytes; (void)s;
  return hipErrorInvalidValue;
}

}  // namespace skv
