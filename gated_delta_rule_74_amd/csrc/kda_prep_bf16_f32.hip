// kda_prep_bf16_f32.hip -- chunk-prep kernels for q/k/v = bf16, g/beta = float
// (the implementation and its description are in kda_prep_impl.h).
#include "kda_prep_impl.h"

namespace kda {
hipError_t launch_prefill_prep_bf16_f32(const PrefillParams &p, hipStream_t s) {
  return prep_dk<bf16, float>(p, s);
}
}  // namespace kda
