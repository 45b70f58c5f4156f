// ParisKV compressed-code retrieval on gfx950 (encode and retrieve).
#include "../../include/sparsekv.h"
#include "skv_internal.h"

extern "C" {

skv_status sparsekv_encode(const skv_codebook* cb, const skv_kv* kv, int32_t b, int32_t t0,
                           int32_t t1, skv_index* index, hipStream_t stream) {
  (void)cb; (void)kv; (void)b; (void)t0; (void)t1; (void)index; (void)stream;
  return SKV_EUNSUPPORTED;
}

skv_status sparsekv_retrieve(const skv_codebook* cb, const skv_index* index, const void* q,
                             int32_t G, float rho, float beta, int32_t k_final, int32_t* idx,
                             int32_t* n_cand, const skv_retrieve_trace* trace, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  (void)cb; (void)index; (void)q; (void)G; (void)rho; (void)beta; (void)k_final; (void)idx;
  (void)n_cand; (void)trace; (void)ws; (void)ws_bytes; (void)stream;
  return SKV_EUNSUPPORTED;
}

size_t sparsekv_retrieve_workspace_size(const skv_index* index, int32_t G, float beta,
                                        int32_t k_final) {
  (void)index; (void)G; (void)beta; (void)k_final;
  return 0;
}

}  // extern "C"
