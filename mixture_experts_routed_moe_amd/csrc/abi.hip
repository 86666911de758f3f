// Host-side plumbing of the C ABI: error reporting and the size helpers.
#include <stdarg.h>
#include <stdio.h>

#include "moe_common.h"

namespace moe {

static thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

}  // namespace moe

extern "C" const char* moe_last_error(void) { return moe::g_last_error; }

extern "C" int moe_abi_version(void) { return 8; }

extern "C" int64_t moe_num_blocks(int64_t numel, int E, int block_m, int padding_m) {
  if (numel < 0 || E < 0 || block_m <= 0 || padding_m <= 0 || padding_m % block_m != 0) return -1;
  return moe::ceil_div(numel, block_m) + static_cast<int64_t>(E) * (padding_m / block_m);
}
