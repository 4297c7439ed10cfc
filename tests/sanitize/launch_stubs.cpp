// Stand-ins for libkda's kernel launchers, linked only into the sanitizer
// build of the validation layer (tests/sanitize/abi_validation.cpp): every
// call there fails validation before reaching a launcher, so none of these
// runs; each would report a launch failure if one did.  max_spec_tokens is
// the draft-length limit the validation layer checks against.
#include <hip/hip_runtime.h>

#include "kda_internal.hpp"

namespace kda {

int device_cus() { return 256; }
int max_spec_tokens() { return 16; }
hipError_t launch_decode(const DecodeArgs&, int, bool, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_prep(const PrefillArgs&, int, int, bool, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_recur(const PrefillArgs&, int, int, bool, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_spec(const SpecArgs&, int, bool, SpecMode, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_epilogue(const EpilogueArgs&, int, bool, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace kda
