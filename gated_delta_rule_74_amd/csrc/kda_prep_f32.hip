// kda_prep_f32.hip -- chunk-prep kernels for q/k/v = float, g/beta = float
// (the implementation and its description are in kda_prep_impl.h).
#include "kda_prep_impl.h"

namespace kda {
hipError_t launch_prefill_prep_f32(const PrefillParams &p, hipStream_t s) {
  return prep_dk<float, float>(p, s);
}
}  // namespace kda
