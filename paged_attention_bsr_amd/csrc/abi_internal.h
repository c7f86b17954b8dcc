// Shared by the two halves of the C ABI: abi_host.cpp (planning and plan
// inspection, host only) and api.cpp (workspace tables, runs, launches).
#pragma once

#include <cstdint>
#include <string>

#include "bsa.h"
#include "planner.h"

struct bsa_plan_s {
  bsa::Plan p;
};

namespace bsa {

// The calling thread's error string (bsa_last_error).
bsa_status_t set_err(bsa_status_t st, const std::string& msg);
void clear_err();

// Device hooks of the host half, defined by api.cpp (abi_host_only.cpp in the
// host-only build the planner's sanitizer tests load):
// the current device's CU count, or an error status with the message set;
bsa_status_t current_device_cus(int32_t* cus);
// drop every workspace binding of a plan about to be destroyed.
void forget_plan(uint64_t plan_id);

}  // namespace bsa
