// kda_prep_bf16_bf16.hip -- chunk-prep kernels for q/k/v = bf16, g/beta = bf16
// (the implementation and its description are in kda_prep_impl.h).
#include "kda_prep_impl.h"

namespace kda {
hipError_t launch_prefill_prep_bf16_bf16(const PrefillParams &p, hipStream_t s) {
  return prep_dk<bf16, bf16>(p, s);
}
}  // namespace kda
