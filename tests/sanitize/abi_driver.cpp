// Drives the C ABI's host code (gated_delta_rule_74_amd/csrc/kda_api.hip)
// under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU:
// every entry point is called with valid and invalid arguments; the kernel
// launchers are replaced here by stubs that record the call and return an
// error, so valid requests end in KDA_EHIP after passing all checks.  Built
// and run by tests/test_sanitizers.py.  Exit status 0 = clean and every
// status as expected.
#include <stdio.h>
#include <stdint.h>

#include "kda.h"
#include "kda_internal.h"

static int launches = 0;
namespace kda {
hipError_t launch_prefill_prep_f32(const PrefillParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
hipError_t launch_prefill_prep_bf16_f32(const PrefillParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
hipError_t launch_prefill_prep_bf16_bf16(const PrefillParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
bool prep_gdn_applies(const PrefillParams &, int) { return false; }
hipError_t launch_prefill_prep_gdn(const PrefillParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
bool prep_d128_applies(const PrefillParams &, int) { return false; }
hipError_t launch_prefill_prep_d128(const PrefillParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
hipError_t launch_state_pass(const PrefillParams &, int, hipStream_t) { ++launches; return hipErrorInvalidValue; }
bool prefill_concurrent_applies(const PrefillParams &, int) { return false; }
hipError_t launch_sync_clear(const PrefillParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
hipError_t launch_state_pass_concurrent(const PrefillParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
hipError_t launch_decode(const DecodeParams &, int, hipStream_t) { ++launches; return hipErrorInvalidValue; }
hipError_t launch_backward(const BwdParams &, int, hipStream_t) { ++launches; return hipErrorInvalidValue; }
bool backward_fits(int, int, int) { return true; }
size_t backward_chunk_floats(int C, int Dk, int Dv) { return (size_t)C * (Dk + Dv); }
hipError_t launch_conv(const ConvParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
hipError_t launch_conv_cache(const ConvParams &, hipStream_t) { ++launches; return hipErrorInvalidValue; }
}  // namespace kda

static int bad = 0;
static void expect(const char *what, kda_status got, kda_status want) {
  if (got != want) {
    printf("%s: status %d, expected %d\n", what, (int)got, (int)want);
    ++bad;
  }
}

int main() {
  // fake, 16-byte aligned device addresses: nothing is ever dereferenced
  char *A = (char *)(uintptr_t)0x100000;
  void *q = A, *k = A + 0x10000, *v = A + 0x20000, *g = A + 0x30000,
       *be = A + 0x40000, *o = A + 0x50000, *ws = A + 0x60000;
  const kda_dtype BF = KDA_BF16, F = KDA_F32;
  const size_t big = (size_t)1 << 40;
  // sizes and strings
  for (int s = 0; s < 6; ++s)
    if (!kda_status_string((kda_status)s)) ++bad;
  if (kda_prefill_workspace_size(1, 8192, 32, 128, 128, 64, BF) == 0) ++bad;
  if (kda_prefill_workspace_size(1, 64, 1, 128, 128, 64, F) !=
      kda_prefill_workspace_size(1, 64, 1, 128, 128, 32, F)) ++bad;
  if (kda_prefill_workspace_size(0, 8, 1, 16, 16, 16, BF) != 0) ++bad;
  if (kda_prefill_workspace_size(1, 0x7fffffff, 1024, 128, 128, 16, BF) == 0) ++bad;
  if (kda_prefill_backward_workspace_size(1, 300, 4, 64, 32, 32, BF) == 0) ++bad;
  // prefill: invalid, unsupported, then valid (reaches the stubbed launch)
  expect("prefill B=0", kda_prefill(q, k, v, BF, g, be, F, nullptr, nullptr, o,
                                    0, 64, 2, 16, 16, 16, 1.f, nullptr, ws, big, nullptr), KDA_EINVAL);
  expect("prefill misaligned", kda_prefill(A + 4, k, v, BF, g, be, F, nullptr, nullptr, o,
                                           1, 64, 2, 16, 16, 16, 1.f, nullptr, ws, big, nullptr), KDA_EINVAL);
  expect("prefill chunk 48", kda_prefill(q, k, v, BF, g, be, F, nullptr, nullptr, o,
                                         1, 64, 2, 16, 16, 48, 1.f, nullptr, ws, big, nullptr), KDA_EUNSUPPORTED);
  expect("prefill ws small", kda_prefill(q, k, v, BF, g, be, F, nullptr, nullptr, o,
                                         1, 64, 2, 16, 16, 16, 1.f, nullptr, ws, 16, nullptr), KDA_EINVAL);
  expect("prefill alias", kda_prefill(q, k, v, BF, g, be, F, nullptr, nullptr, q,
                                      1, 64, 2, 16, 16, 16, 1.f, nullptr, ws, big, nullptr), KDA_EINVAL);
  expect("prefill valid", kda_prefill(q, k, v, BF, g, be, F, nullptr, nullptr, o,
                                      2, 1000, 3, 128, 64, 64, 0.5f, nullptr, ws, big, nullptr), KDA_EHIP);
  expect("prefill head gate", kda_prefill(q, k, v, BF, g, be, (kda_dtype)(F | KDA_GATE_HEAD),
                                          nullptr, nullptr, o, 1, 77, 2, 128, 128, 64, 1.f,
                                          nullptr, ws, big, nullptr), KDA_EHIP);
  kda_conv_desc cd = {q, k, v, (const float *)g, (const float *)be, (const float *)ws, 4, 1, 1e-6f};
  expect("prefill conv", kda_prefill(nullptr, nullptr, nullptr, BF, g, be, F, nullptr, nullptr, o,
                                     1, 100, 2, 64, 64, 32, 1.f, &cd, A + 0x70000, big, nullptr), KDA_EHIP);
  cd.width = 1;
  expect("prefill conv width 1", kda_prefill(nullptr, nullptr, nullptr, BF, g, be, F, nullptr, nullptr, o,
                                             1, 100, 2, 64, 64, 32, 1.f, &cd, A + 0x70000, big, nullptr), KDA_EINVAL);
  // the no-allocation prefill: oversize is refused before anything else
  expect("noalloc oversize", kda_prefill_noalloc(q, k, v, BF, g, be, F, nullptr, nullptr, o,
                                                 1, 2048, 32, 128, 128, 64, 1.f, nullptr, nullptr), KDA_ENOSPACE);
  expect("noalloc invalid", kda_prefill_noalloc(q, k, v, BF, g, be, F, nullptr, nullptr, o,
                                                1, 0, 32, 128, 128, 64, 1.f, nullptr, nullptr), KDA_EINVAL);
  // the two phases, the backward, decode, verify and the conv prologue
  expect("prep", kda_prefill_chunk_prep(q, k, v, BF, g, be, BF, 1, 65, 2, 32, 32, 16, 1.f,
                                        nullptr, ws, big, nullptr), KDA_EHIP);
  expect("state", kda_prefill_state_pass(BF, nullptr, nullptr, o, 1, 65, 2, 32, 32, 16,
                                         ws, big, nullptr), KDA_EHIP);
  expect("bwd alias", kda_prefill_backward(q, k, v, BF, g, be, F, nullptr, o, nullptr,
                                           A + 0x80000, A + 0x80000, A + 0x90000, A + 0xa0000,
                                           A + 0xb0000, nullptr, 1, 64, 2, 16, 16, 16, 1.f,
                                           ws, big, nullptr), KDA_EINVAL);
  expect("bwd valid", kda_prefill_backward(q, k, v, BF, g, be, F, nullptr, o, nullptr,
                                           A + 0x80000, A + 0x88000, A + 0x90000, A + 0xa0000,
                                           A + 0xb0000, nullptr, 1, 300, 2, 64, 32, 32, 1.f,
                                           ws, big, nullptr), KDA_EHIP);
  float *st = (float *)(A + 0xc0000);
  expect("decode valid", kda_decode_step(q, k, v, BF, g, be, BF, st, o, 5, 3, 128, 64, 1.f,
                                         nullptr), KDA_EHIP);
  expect("decode dims", kda_decode_step(q, k, v, BF, g, be, BF, st, o, 5, 3, 100, 64, 1.f,
                                        nullptr), KDA_EUNSUPPORTED);
  expect("tokens L=0", kda_decode_tokens(q, k, v, BF, g, be, BF, st, st, nullptr, o, 4, 0, 2,
                                         64, 64, 1.f, nullptr, nullptr, nullptr, nullptr), KDA_EINVAL);
  cd.width = 4;
  expect("tokens conv", kda_decode_tokens(nullptr, nullptr, nullptr, BF, g, be, BF, st, st,
                                          nullptr, o, 4, 2, 2, 64, 64, 1.f, &cd,
                                          (float *)(A + 0xd0000), nullptr, nullptr), KDA_EHIP);
  expect("conv prologue", kda_conv_prologue(q, k, v, BF, (const float *)g, (const float *)be,
                                            (const float *)ws, 3, nullptr, A + 0xe0000,
                                            A + 0xe8000, A + 0xf0000, 2, 50, 3, 32, 16, 1,
                                            1e-6f, nullptr), KDA_EHIP);
  expect("conv width 5", kda_conv_prologue(q, k, v, BF, (const float *)g, (const float *)be,
                                           (const float *)ws, 5, nullptr, A + 0xe0000,
                                           A + 0xe8000, A + 0xf0000, 2, 50, 3, 32, 16, 1,
                                           1e-6f, nullptr), KDA_EUNSUPPORTED);
  printf("C ABI under sanitizers: %d mismatches, %d stubbed launches\n", bad,
         launches);
  return bad == 0 && launches > 0 ? 0 : 1;
}
