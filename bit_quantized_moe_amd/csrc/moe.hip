// MoE layer entry points (placeholder until the grouped GEMMs land).
#include "common.h"

extern "C" size_t bqm_moe_workspace_size(const bqm_moe_desc *) { return 0; }
extern "C" bqm_status bqm_moe_fwd(const bqm_moe_desc *, const uint16_t *, const int32_t *, const float *,
                                  uint16_t *, void *, size_t, void *) {
  return bqm::fail(BQM_ERR_UNSUPPORTED, "bqm_moe_fwd: not built yet");
}
extern "C" bqm_status bqm_moe_dgrad(const bqm_moe_desc *, const uint16_t *, void *, size_t, uint16_t *,
                                    float *, void *) {
  return bqm::fail(BQM_ERR_UNSUPPORTED, "bqm_moe_dgrad: not built yet");
}
extern "C" bqm_status bqm_lora_grad(const bqm_moe_desc *, void *, size_t, float *, float *, float *, float *,
                                    void *) {
  return bqm::fail(BQM_ERR_UNSUPPORTED, "bqm_lora_grad: not built yet");
}
