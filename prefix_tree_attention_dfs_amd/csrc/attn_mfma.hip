// bf16 MFMA tree attention (head dim 128) -- placeholder until the kernels land.
#include "device.h"
#include "kernels.h"

bool mfma_attn_supported(const AttnGeom&, const PlanPtrs&) { return false; }
int launch_fwd_mfma(const void*, const void*, const void*, void*, float*, const PlanPtrs&, const AttnGeom&, bool,
                    hipStream_t) {
  return -1;
}
int launch_bwd_mfma(const void*, const void*, const void*, const void*, const float*, const float*, float*, void*,
                    void*, bool, const PlanPtrs&, const AttnGeom&, bool, hipStream_t) {
  return -1;
}
