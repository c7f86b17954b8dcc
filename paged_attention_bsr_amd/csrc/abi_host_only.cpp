// Device hooks for a host-only build of the planner and the host half of the
// C ABI (planner.cpp + abi_host.cpp + this file, no HIP): the library the
// planner tests load under AddressSanitizer and UndefinedBehaviorSanitizer.
// Plans there need num_cus > 0; there are no workspace bindings to forget.
#include "abi_internal.h"

namespace bsa {

bsa_status_t current_device_cus(int32_t*) {
  return set_err(BSA_ERR_UNSUPPORTED, "host-only build: pass num_cus > 0 to plan without a GPU");
}

void forget_plan(uint64_t) {}

}  // namespace bsa
