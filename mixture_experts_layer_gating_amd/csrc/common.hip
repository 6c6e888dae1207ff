// Error state and version of the library.
#include "moe_internal.h"

namespace moe {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

moe_status check_launch(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error(std::string(what) + ": " + hipGetErrorString(err));
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // namespace moe

extern "C" const char* moe_last_error(void) { return moe::g_last_error.c_str(); }

extern "C" const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }
