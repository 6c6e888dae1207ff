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

extern "C" moe_status moe_index_errors(unsigned int* mask, int clear, moe_stream_t stream) {
  using namespace moe;
  clear_error();
  MOE_REQUIRE(mask != nullptr, MOE_ERR_INVALID_ARG, "moe_index_errors: null mask");
  unsigned int bits = 0;
  hipStream_t st = as_stream(stream);
  const bool c = clear != 0;
  if (moe_status s = index_record_route(st, &bits, c)) return s;
  if (moe_status s = index_record_count(st, &bits, c)) return s;
  if (moe_status s = index_record_move(st, &bits, c)) return s;
  if (moe_status s = index_record_gemm(st, &bits, c)) return s;
  *mask = bits;
  return MOE_OK;
}
